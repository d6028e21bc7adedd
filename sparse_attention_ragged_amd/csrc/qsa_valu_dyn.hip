// Gather-attention kernel on wavefront dot products (groups of 1, 2 or 4 query heads
// per kv head), dynamically scheduled.
//
// The work of every (query row, kv head) key list ("QSASparseAttentionRaggedPaged":
// token_indices up to counts; "Struct_msa_attention_ragged_paged": the positions of
// the listed blocks up to the row's position; "latent_sparse_attention_ragged_paged":
// window positions, then listed compressed entries) is cut into units of CK
// consecutive keys, and each unit leaves an (m, l, acc) partial that the split-K
// combine kernel merges ("Struct_msa_attention_ragged_paged" design notes: decode over
// partitioned KV bands, then a reduction kernel). Units are numbered (row, kv head,
// part), part fastest.
//
// A persistent grid (one workgroup per CU) takes units as it goes: the first two
// units of workgroup w are w and w + grid, every further one comes from a counter in
// the workspace. On this GPU equal static shares of a gather finish up to a fifth
// apart (whole XCDs and the younger of two wavefronts sharing a SIMD run slower, and
// which ones changes from launch to launch); taking units as they free up evens that
// out.
//
// A workgroup is two streams of streaming wavefronts plus one control wavefront:
//  * stream 0 is wavefronts 0-3 and stream 1 wavefronts 4-6. The second wavefront on
//    a SIMD streams about a fifth slower than the first, so the two kinds do not share
//    units: each stream runs its own sequence of units, and the slower one simply
//    takes fewer of them from the counter;
//  * a streaming wavefront runs the address pipeline and team arithmetic of the
//    statically scheduled kernel (qsa_valu_core.hpp) over one continuous stream of key
//    batches: the pipeline does not restart between units, the stages of a batch read
//    the context of the unit the batch belongs to. At the end of a unit the wavefront
//    merges its teams, leaves its state in the unit's LDS merge slot, counts itself
//    done there and goes on without waiting for the other wavefronts;
//  * the control wavefront keeps, per stream, a ring of unit contexts (row, kv head,
//    list length, sequence, position and the q rows, loaded in one round trip): when
//    every wavefront of a stream is done with its oldest unit, it merges their states
//    into the unit's partial, claims a new unit and publishes its context in the freed
//    slot (a sequence number written last), one slot ahead of the stream's first stage.
//    A streaming wavefront waits only when it reaches a slot that is not published
//    yet; that wait always ends, because the slot it waits for is freed by wavefronts
//    that are not waiting (a unit spans enough key batches for the ring to hold every
//    slot a wavefront's pipeline can reach, so a waiting wavefront is itself past the
//    stream's oldest unit).
//    Units that start past their row's list length are written as empty partials
//    without being streamed.
// No workgroup barrier is used after the first one: LDS operations of one wavefront
// take effect in order, which orders each state before its done count and each
// context before its sequence number.
//
// The counter must be zero when a launch starts; the combine kernel that follows
// every launch resets it (so a workspace is zero-filled once, before its first use).
#include "qsa_valu_core.hpp"

namespace qsa {

namespace {

constexpr int kDynThreads = 64 * 8;
constexpr int kCtrlWave = 7;
constexpr uint32_t kNoUnit = 0xffffffffu;

__device__ __forceinline__ int stream_of(int wave) { return wave < 4 ? 0 : 1; }
__device__ __forceinline__ int stream_waves(int x) { return x == 0 ? 4 : 3; }

// Context of one unit of a stream.
struct SlotCtx {
    uint32_t unit;      // kNoUnit: the stream ends at this slot
    int32_t r;          // query row
    int32_t g;          // kv head
    int32_t b;          // sequence of the row
    int64_t n;          // list length of the row
    int64_t pos;        // position of the row (block-sparse and latent lists)
};

// LDS of the dynamically scheduled kernel: per stream a ring of RING unit slots.
template <int G, int D, int QBYTES, int RING>
struct DynLds {
    SlotCtx ctx[2][RING];
    uint32_t seq[2][RING];              // slot number + 1 once its context is published
    uint32_t done[2][RING];             // streaming wavefronts done with the slot
    uint32_t e_slot[2];                 // newest slot the stream's first stage has entered
    float ml[2][RING][4][G][2];         // their (reference, sum) per q head
    float acc[2][RING][4][G][D];        // their accumulators
    char q[2][RING][QBYTES];
};

__device__ __forceinline__ int64_t uniform64(int64_t v)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// A slot context read from LDS as wavefront-uniform values.
__device__ __forceinline__ SlotCtx read_ctx(const SlotCtx &c)
{
    SlotCtx u;
    u.unit = __builtin_amdgcn_readfirstlane(c.unit);
    u.r = __builtin_amdgcn_readfirstlane(c.r);
    u.g = __builtin_amdgcn_readfirstlane(c.g);
    u.b = __builtin_amdgcn_readfirstlane(c.b);
    u.n = uniform64(c.n);
    u.pos = uniform64(c.pos);
    return u;
}

__device__ __forceinline__ uint32_t lds_load(const uint32_t *a)
{
    return __builtin_amdgcn_readfirstlane(__hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
}

template <int DT, int D, int G>
constexpr int dyn_ring()
{
    // as many slots as fit 150 KB of LDS, 2 to 4
    constexpr int qb = G * D * Elem<DT>::bytes;
    constexpr int per = (int)sizeof(SlotCtx) + 8 + 4 * G * 2 * 4 + 4 * G * D * 4 + qb;
    constexpr int r = 150 * 1024 / (2 * per);
    return r > 4 ? 4 : r;
}

template <int DT, int D, int G, int LIST>
__global__ void __launch_bounds__(kDynThreads) gather_valu_dyn_kernel(GatherParams p)
{
    constexpr int U = 2;
    using Core = ValuCore<DT, D, G, U>;
    constexpr int EB = Core::EB;
    constexpr int CPL = Core::CPL;
    constexpr int EPC = Core::EPC;
    constexpr int TL = Core::TL;
    constexpr int TPW = Core::TPW;
    constexpr int QBYTES = G * D * EB;           // q rows of one (row, kv head)
    constexpr int RING = dyn_ring<DT, D, G>();
    static_assert(QBYTES % 16 == 0, "q rows must be whole 16-byte chunks");
    static_assert(RING >= 2, "the unit ring needs two slots per stream");
    // a unit spans at least kMinBatches key batches: a wavefront's first stage runs
    // three batches ahead of its last, so it is at most ceil(3 / kMinBatches) units
    // ahead, which the ring must hold (RING - 1 >= ceil(3 / kMinBatches))
    constexpr int kMinBatches = RING >= 4 ? 1 : RING == 3 ? 2 : 3;
    using Lds = DynLds<G, D, QBYTES, RING>;
    __shared__ Lds L;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t C = (uint32_t)p.num_splits;             // units per (row, kv head)
    const int64_t CK = p.split_keys;                       // keys per unit
    const uint32_t Hkv = (uint32_t)p.num_kv_heads;
    const uint32_t units = (uint32_t)p.total_q * Hkv * C;  // < 2^31 (checked by the planner)
    const uint32_t grid = gridDim.x;

    // every ring slot starts as an empty context with in-range fields, so that no
    // stage can ever address memory from a context that was never published
    if (tid < 2 * RING) {
        L.seq[tid / RING][tid % RING] = 0u;
        L.done[tid / RING][tid % RING] = 0u;
        L.ctx[tid / RING][tid % RING] = SlotCtx{kNoUnit, 0, 0, 0, 0, 0};
    }
    if (tid < 2)
        L.e_slot[tid] = 0u;
    __syncthreads();

    if (wave == kCtrlWave) {
        // ------------------------------------------------ control wavefront
        // one unit from the counter (one atomic, by lane 0)
        auto grab = [&]() -> uint32_t {
            uint32_t t = 0;
            if (lane == 0)
                t = atomicAdd(p.sched_counter, 1u);
            t = __builtin_amdgcn_readfirstlane(t) + 2u * grid;
            return t < units ? t : kNoUnit;
        };
        // the partial of a unit that has no keys
        auto write_empty = [&](uint32_t unit) {
            const uint32_t item = unit / C, part = unit % C;
            const int64_t r = item / Hkv, g = item % Hkv;
            const int64_t srh0 = ((int64_t)part * p.total_q + r) * p.num_q_heads + g * G;
            for (int i = lane; i < G * D / 4; i += 64)
                *reinterpret_cast<float4 *>(p.ws_acc + srh0 * D + 4 * i) = make_float4(0.f, 0.f, 0.f, 0.f);
            if (lane < G) {
                p.ws_ml[(srh0 + lane) * 2] = kNoKey;
                p.ws_ml[(srh0 + lane) * 2 + 1] = 0.f;
            }
        };
        // publish slot k of stream x for `unit`, first skipping (and writing empty)
        // units that start past their row's list length; returns the unit the slot
        // holds. The list length, the sequence offsets (and positions) and the q rows
        // of a unit are loaded together: one memory round trip per context.
        constexpr int QL = (QBYTES + 1023) / 1024;     // 16-byte q loads per lane
        auto publish = [&](int x, int k, uint32_t unit) -> uint32_t {
            const int e = k % RING;
            SlotCtx c{kNoUnit, 0, 0, 0, 0, 0};
            while (unit != kNoUnit) {
                const uint32_t item = unit / C, part = unit % C;
                const int32_t r = (int32_t)(item / Hkv);
                const int32_t g = (int32_t)(item % Hkv);
                const int64_t n_raw = key_list_length_v<LIST>(p, r);
                const bool small = p.batch <= 64;
                uint32_t lo = 0xffffffffu, hi = 0u, cl = 0u;
                if (small && lane < p.batch) {
                    lo = p.row_off[lane];
                    hi = p.row_off[lane + 1];
                    if constexpr (LIST != KEYS_TOKEN_INDICES)
                        cl = p.cache_lengths[lane];
                }
                const char *qsrc = static_cast<const char *>(p.q) + ((int64_t)r * p.num_q_heads + (int64_t)g * G) * D * EB;
                u32x4 qv[QL];
#pragma unroll
                for (int i = 0; i < QL; ++i) {
                    const int o = 16 * lane + 1024 * i;
                    qv[i] = o < QBYTES ? ldg16(qsrc + o) : u32x4{0, 0, 0, 0};
                }
                const int64_t n = uniform64(n_raw);
                if ((int64_t)part * CK < n) {
                    c.unit = unit;
                    c.r = r;
                    c.g = g;
                    c.n = n;
                    if (small) {
                        const unsigned long long m = __ballot(lo <= (uint32_t)r && (uint32_t)r < hi);
                        // rows past the last offset belong to the last sequence
                        const int w = m ? __ffsll((long long)m) - 1 : p.batch - 1;
                        const uint32_t lo_w = (uint32_t)__shfl((int)lo, w), cl_w = (uint32_t)__shfl((int)cl, w);
                        c.b = w;
                        c.pos = LIST == KEYS_TOKEN_INDICES ? 0
                                                           : uniform64((int64_t)cl_w + ((int64_t)r - (int64_t)lo_w));
                    } else {
                        int64_t pos = 0;
                        c.b = find_seq_pos_wave(p.row_off, LIST == KEYS_TOKEN_INDICES ? nullptr : p.cache_lengths,
                                                p.batch, (uint32_t)r, pos);
                        c.pos = uniform64(pos);
                    }
#pragma unroll
                    for (int i = 0; i < QL; ++i) {
                        const int o = 16 * lane + 1024 * i;
                        if (o < QBYTES)
                            *reinterpret_cast<u32x4 *>(&L.q[x][e][o]) = qv[i];
                    }
                    break;
                }
                write_empty(unit);
                unit = grab();
            }
            if (lane == 0) {
                L.ctx[x][e] = c;
                L.done[x][e] = 0u;
            }
            asm volatile("" ::: "memory");
            if (lane == 0)
                __hip_atomic_store(&L.seq[x][e], (uint32_t)k + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            return c.unit;
        };
        // merge the states of stream x's wavefronts for slot k into the unit's partial
        auto write_partial = [&](int x, int k) {
            const int e = k % RING;
            const int nw = stream_waves(x);
            const SlotCtx c = read_ctx(L.ctx[x][e]);
            const int64_t part = c.unit % C;
            const int64_t srh0 = (part * p.total_q + c.r) * p.num_q_heads + (int64_t)c.g * G;
            for (int i = lane; i < G * D / 4; i += 64) {
                const int h = (4 * i) / D, d = 4 * i - h * D;
                float M = kNoKey;
                for (int w = 0; w < nw; ++w)
                    M = fmaxf(M, L.ml[x][e][w][h][0]);
                float Ls = 0.f;
                float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
                for (int w = 0; w < nw; ++w) {
                    const float cw = __builtin_amdgcn_exp2f(L.ml[x][e][w][h][0] - M);
                    const float4 a = *reinterpret_cast<const float4 *>(&L.acc[x][e][w][h][d]);
                    Ls += cw * L.ml[x][e][w][h][1];
                    A.x += cw * a.x;
                    A.y += cw * a.y;
                    A.z += cw * a.z;
                    A.w += cw * a.w;
                }
                *reinterpret_cast<float4 *>(p.ws_acc + (srh0 + h) * D + d) = A;
                if (d == 0) {
                    p.ws_ml[(srh0 + h) * 2] = M;
                    p.ws_ml[(srh0 + h) * 2 + 1] = Ls;
                }
            }
        };

        int oldest[2] = {0, 0};        // oldest slot not merged yet
        int next[2] = {0, 0};          // next slot to publish
        bool ended[2] = {false, false};   // the stream's last published slot is empty
        auto publish_next = [&](int x, uint32_t unit) {
            const uint32_t u = publish(x, next[x], unit);
            ++next[x];
            ended[x] = u == kNoUnit;
        };
        // Each stream holds its slot in progress and one more: a unit is claimed and
        // published when the stream's first stage enters the newest published slot.
        // Claiming further ahead would leave a slow stream with several units queued
        // when the counter runs out.
        publish_next(0, blockIdx.x);
        publish_next(1, blockIdx.x + grid < units ? blockIdx.x + grid : kNoUnit);
        for (int x = 0; x < 2; ++x)
            if (!ended[x])
                publish_next(x, grab());
        for (;;) {
            bool busy = false, progressed = false;
            for (int x = 0; x < 2; ++x) {
                const int k = oldest[x];
                if (ended[x] && k == next[x] - 1)
                    continue;                    // only the empty end slot is left
                busy = true;
                const int e = k % RING;
                if (lds_load(&L.done[x][e]) == (uint32_t)stream_waves(x)) {
                    asm volatile("" ::: "memory");
                    write_partial(x, k);
                    ++oldest[x];
                    progressed = true;
                }
                if (!ended[x] && next[x] <= (int)lds_load(&L.e_slot[x]) + 1 && next[x] < oldest[x] + RING) {
                    publish_next(x, grab());
                    progressed = true;
                }
            }
            if (!busy)
                break;
            if (!progressed)
                __builtin_amdgcn_s_sleep(8);
        }
        return;
    }

    // ---------------------------------------------------- streaming wavefronts
    const int x = stream_of(wave);
    const int wx = x == 0 ? wave : wave - 4;     // wavefront within the stream
    const int NK = stream_waves(x) * TPW;        // key slots of the stream
    const int ln = tid % TL;
    const int ks = lane / TL;                    // key slot (team) within the wavefront
    const int64_t per_batch = (int64_t)NK * U;
    const char *dummy = static_cast<const char *>(p.q);   // a readable row for absent keys
    const int64_t vdelta = LIST == KEYS_LATENT ? 0 : (int64_t)p.kv.plane_stride_b;

    // wait until slot k of this stream is published (the wait always ends: see above)
    auto wait_slot = [&](int k) {
        while (lds_load(&L.seq[x][k % RING]) != (uint32_t)k + 1u)
            __builtin_amdgcn_s_sleep(1);
        asm volatile("" ::: "memory");
    };
    wait_slot(0);
    if (read_ctx(L.ctx[x][0]).unit == kNoUnit)
        return;

    // Per-stage position in the stream (slot k, batch lb of the slot's nbs batches)
    // and the fields of the slot's context the stage uses, read from LDS on entering a
    // slot (the first stage waits for the slot to be published; the later stages
    // enter it after the first, and a slot is not reused before every wavefront of
    // the stream is done with it). A slot runs ceil(keys / batch) batches but at least
    // kMinBatches. The empty slot that ends the stream is absorbing: a stage that
    // reaches it stays there with no keys and reads no further slot (the stages run up
    // to three batches ahead of the fold, and the slots past the end were never
    // published).
    struct StageE { int k, lb, nbs; bool live; int32_t r, g; int64_t j0, j1; };
    struct StageP { int k, lb, nbs; int32_t b; int64_t j0, j1, pos; };
    struct StageR { int k, lb, nbs; int32_t g; };
    struct StageC { int k, lb, nbs; };
    auto range = [&](const SlotCtx &c, int64_t &j0, int64_t &j1) -> int {
        if (c.unit == kNoUnit) {
            j0 = j1 = 0;
            return 0x7fffffff;          // absorbing: the stage never leaves this slot
        }
        j0 = (int64_t)(c.unit % C) * CK;
        j1 = c.n < j0 + CK ? c.n : j0 + CK;
        const int nb = (int)((j1 - j0 + per_batch - 1) / per_batch);
        return nb > kMinBatches ? nb : kMinBatches;
    };
    StageE se{0, 0, 0, true, 0, 0, 0, 0};
    StageP sp{0, 0, 0, 0, 0, 0, 0};
    StageR sr{0, 0, 0, 0};
    StageC sc{0, 0, 0};

    struct Entries { int32_t raw[U]; };
    struct Pages { KeyPos k[U]; int32_t slot[U]; uint32_t page[U]; };
    using Rows = typename Core::Rows;

    auto key_index = [&](int64_t j0, int lb, int u) -> int64_t {
        return j0 + lb * per_batch + u * NK + wx * TPW + ks;
    };
    auto load_entries = [&](Entries &E) {
        if (se.lb == 0) {
            if (se.live) {
                if (lane == 0)
                    __hip_atomic_fetch_max(&L.e_slot[x], (uint32_t)se.k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                wait_slot(se.k);
                const SlotCtx c = read_ctx(L.ctx[x][se.k % RING]);
                se.live = c.unit != kNoUnit;
                se.r = c.r;
                se.g = c.g;
                se.nbs = range(c, se.j0, se.j1);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t jj = key_index(se.j0, se.lb, u);
            E.raw[u] = *entry_ptr<LIST>(p, se.r, se.g, jj, jj < se.j1);
        }
        if (++se.lb == se.nbs) {
            se.lb = 0;
            ++se.k;
        }
    };
    auto load_pages = [&](const Entries &E, Pages &P) {
        if (sp.lb == 0) {
            const SlotCtx c = read_ctx(L.ctx[x][sp.k % RING]);
            sp.b = c.b;
            sp.pos = c.pos;
            sp.nbs = range(c, sp.j0, sp.j1);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t jj = key_index(sp.j0, sp.lb, u);
            P.k[u] = key_pos<LIST>(p, sp.pos, jj, E.raw[u], jj < sp.j1);
            P.page[u] = *page_entry_ptr<LIST>(p, sp.b, P.k[u], P.slot[u]);
        }
        if (++sp.lb == sp.nbs) {
            sp.lb = 0;
            ++sp.k;
        }
    };
    auto load_rows = [&](const Pages &P, Rows &R) {
        if (sr.lb == 0) {
            const SlotCtx c = read_ctx(L.ctx[x][sr.k % RING]);
            sr.g = c.g;
            int64_t j0, j1;
            sr.nbs = range(c, j0, j1);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            bool ok;
            const char *a = row_address<EB, LIST>(p, P.k[u], P.page[u], P.slot[u], sr.g, dummy, ok);
            R.ok[u] = ok;
            const char *base = ok ? a : dummy;
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                R.k[u][c] = ldg16(base + (int64_t)Core::chunk_elem(c, ln) * EB);
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                R.v[u][c] = ldg16((ok ? a + vdelta : dummy) + (int64_t)Core::chunk_elem(c, ln) * EB);
        }
        if (++sr.lb == sr.nbs) {
            sr.lb = 0;
            ++sr.k;
        }
    };

    typename Core::Q q;
    Core st;
    st.reset();
    // fold one batch; at the end of a slot leave the wavefront's state in the slot's
    // merge area and count it done. Returns false when the stream has ended.
    auto consume = [&](const Rows &R) -> bool {
        const int e = sc.k % RING;
        if (sc.lb == 0) {
            int64_t j0, j1;
            sc.nbs = range(read_ctx(L.ctx[x][e]), j0, j1);
            const char *qs = L.q[x][e];
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    q.raw[h][c] = *reinterpret_cast<const u32x4 *>(qs + (h * D + Core::chunk_elem(c, ln)) * EB);
            Core::widen_q(q);
        }
        st.consume(R, q, p.scale_log2);
        if (++sc.lb < sc.nbs)
            return true;
        st.merge_teams_lean();
        if (ks == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                if (ln == 0) {
                    L.ml[x][e][wx][h][0] = st.m[h];
                    L.ml[x][e][wx][h][1] = st.l[h];
                }
#pragma unroll
                for (int c = 0; c < CPL; ++c)
#pragma unroll
                    for (int i = 0; i < EPC; i += 4)
                        *reinterpret_cast<float4 *>(&L.acc[x][e][wx][h][Core::chunk_elem(c, ln) + i]) =
                            make_float4(st.acc[h][c * EPC + i], st.acc[h][c * EPC + i + 1],
                                        st.acc[h][c * EPC + i + 2], st.acc[h][c * EPC + i + 3]);
            }
        }
        st.reset();
        asm volatile("" ::: "memory");
        if (lane == 0)
            __hip_atomic_fetch_add(&L.done[x][e], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        sc.lb = 0;
        ++sc.k;
        // the next slot was published before the first stage entered it
        return read_ctx(L.ctx[x][sc.k % RING]).unit != kNoUnit;
    };

    // iteration i issues entries(i+2), pages(i+1), rows(i) and folds rows(i-1), over
    // the whole stream; register sets alternate between even and odd iterations
    Entries E0, E1;
    Pages P0, P1;
    Rows R0, R1;
    load_entries(E0);
    load_entries(E1);
    load_pages(E0, P0);
    load_entries(E0);
    load_pages(E1, P1);
    load_rows(P0, R0);
    load_entries(E1);
    load_pages(E0, P0);
    load_rows(P1, R1);
    bool more = consume(R0);
    while (more) {
        load_entries(E0);
        load_pages(E1, P1);
        load_rows(P0, R0);
        if (!consume(R1))
            break;
        load_entries(E1);
        load_pages(E0, P0);
        load_rows(P1, R1);
        more = consume(R0);
    }
}

template <int DT, int D, int G, int LIST>
int launch_valu_dyn(const GatherParams &p, void *stream)
{
    if (p.sched_grid <= 0)
        return 0;
    hipLaunchKernelGGL((gather_valu_dyn_kernel<DT, D, G, LIST>), dim3((unsigned)p.sched_grid), dim3(kDynThreads), 0,
                       static_cast<hipStream_t>(stream), p);
    return (int)hipGetLastError();
}

template <int DT, int D, int LIST>
int launch_valu_dyn_g(const GatherParams &p, void *stream)
{
    switch (p.group) {
    case 1: return launch_valu_dyn<DT, D, 1, LIST>(p, stream);
    case 2: return launch_valu_dyn<DT, D, 2, LIST>(p, stream);
    case 4: return launch_valu_dyn<DT, D, 4, LIST>(p, stream);
    default: return (int)hipErrorInvalidValue;
    }
}

template <int DT, int LIST>
int launch_valu_dyn_d(const GatherParams &p, void *stream)
{
    switch (p.head_dim) {
    case 64: return launch_valu_dyn_g<DT, 64, LIST>(p, stream);
    case 128: return launch_valu_dyn_g<DT, 128, LIST>(p, stream);
    case 256: return launch_valu_dyn_g<DT, 256, LIST>(p, stream);
    default: return (int)hipErrorInvalidValue;
    }
}

template <int LIST>
int launch_valu_dyn_t(const GatherParams &p, void *stream)
{
    switch (p.dtype) {
    case QSA_F32: return launch_valu_dyn_d<QSA_F32, LIST>(p, stream);
    case QSA_BF16: return launch_valu_dyn_d<QSA_BF16, LIST>(p, stream);
    case QSA_FP8_E4M3: return launch_valu_dyn_d<QSA_FP8_E4M3, LIST>(p, stream);
    default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace

int launch_gather_valu_dyn(const GatherParams &p, void *stream)
{
    if (!p.sched_counter || p.sched_bpu < 3 || p.num_splits < 1 || !p.ws_acc || !p.ws_ml)
        return (int)hipErrorInvalidValue;
    switch (p.list_kind) {
    case KEYS_TOKEN_INDICES: return launch_valu_dyn_t<KEYS_TOKEN_INDICES>(p, stream);
    case KEYS_BLOCKS: return launch_valu_dyn_t<KEYS_BLOCKS>(p, stream);
    case KEYS_LATENT: return launch_valu_dyn_t<KEYS_LATENT>(p, stream);
    default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace qsa
