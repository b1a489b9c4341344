// Causal ELU+1 linear attention, chunked prefill on gfx950.
//
// The method ("AIGC 基本功｜线性、循环与记忆架构-LinearMem", §03): with
// phi = ELU+1, S_t = S_{t-1} + phi(k_t) v_t^T, z_t = z_{t-1} + phi(k_t) and the
// write-then-read output o_t^T = phi(q_t)^T S_t / (phi(q_t)^T z_t + eps).
//
// Chunked form (a chunk of C = 64 tokens, state (S, z) at the chunk start):
//   P     = tril(phi(Q_c) phi(K_c)^T)                 (diagonal kept: write-then-read)
//   num   = P V_c + phi(Q_c) S,  den = P 1 + phi(Q_c) z + eps,  O_c = num / den
//   S    += phi(K_c)^T V_c,      z  += phi(K_c)^T 1
// Only the state crosses a chunk boundary ("手撕：递推与记忆模型", "Chunked
// scan"; the chunkwise small-attention-plus-state form of "线性注意力与 SSM"
// §3).  The sum z rides along as one extra 16-column tile: V is extended with
// a block of ones and S with 16 copies of z, so the denominator comes out of
// the same MFMA chain as the numerator, in the same registers.
//
// Sequence parallelism: each head's tokens are cut into G segments, one
// workgroup each.  Because the state update is additive, the state entering
// segment g is S0 + sum_{g' < g} (segment sum of g'); workgroups find it by
// decoupled look-back over their predecessors' published sums (one launch,
// after a launch that clears the look-back flags).
#include "common.hpp"
#include "kernels.hpp"

namespace la {

namespace {

constexpr int CH = kChunk;
constexpr int NTHR = 256;  // four waves; wave w owns query rows 16w..16w+15

template <typename TIn, int DK, int DV>
struct Layout {
    using op = typename Mma<TIn>::op_t;
    static constexpr int PAD = 16 / sizeof(op);
    static constexpr int LQ = DK + PAD;          // rows of phi(Q), phi(K) and S^T: k = dk
    static constexpr int LV = DV + PAD;          // rows of V and of the output tile
    static constexpr int NCT = DV / 16 + 1;      // value column tiles + the ones/z tile
    static constexpr int RTW = DK / 64;          // dk row tiles per wave (4 waves)
    static constexpr int E = DK * DV + DK;       // floats per (head, segment) state
};

// ------------------------------------------------------------- la_fused
//
// Single pass with decoupled look-back.  Workgroup b handles segment
// b / HT of head b % HT (segment-major order, so every predecessor segment of
// a head has a smaller block index and was dispatched earlier):
//   1. sum phi(K)^T [V | 1] over its segment (its aggregate);
//   2. publish the aggregate (flag 1); find the state entering the segment by
//      walking back over predecessors: an inclusive state (flag 2) ends the
//      walk, an aggregate is added and the walk continues;
//   3. publish its own inclusive state (flag 2);
//   4. run the chunk loop from that state, writing the outputs.
// Published states are written and read with relaxed agent-scope atomics
// (coherent across the chip's L2s); the flag is stored only after the data
// stores have completed.  Every wait is bounded: a workgroup that times out
// recomputes its incoming state from the inputs (sum over all earlier
// tokens), so progress never depends on the dispatch order.

enum : int { kFlagNone = 0, kFlagAggregate = 1, kFlagInclusive = 2 };
constexpr int kPollLimit = 4000;  // polls of one window before giving up (~ms)

__device__ __forceinline__ int load_flag(const int* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_flag(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// acc += phi(K)^T [V | 1] over tokens [t0, t1), next chunk's loads in flight.
template <typename TIn, int DK, int DV>
__device__ __forceinline__ void accumulate_kv(const TIn* kh, const TIn* vh, int t0, int t1,
                                              v4f (&acc)[Layout<TIn, DK, DV>::RTW][Layout<TIn, DK, DV>::NCT],
                                              typename Mma<TIn>::op_t* Ks, typename Mma<TIn>::op_t* Vs,
                                              int tid) {
    using M = Mma<TIn>;
    using LY = Layout<TIn, DK, DV>;
    const int lane = tid & 63, w = wave_id(tid);
    if (t0 >= t1) return;
    ChunkRegs<TIn, DK, NTHR> kr;
    ChunkRegs<TIn, DV, NTHR> vr;
    kr.load(kh, t0, min(CH, t1 - t0), tid);
    vr.load(vh, t0, min(CH, t1 - t0), tid);
    for (int c0 = t0; c0 < t1; c0 += CH) {
        const int n = min(CH, t1 - c0);
        stage_rows<TIn, DK, NTHR>(kr, true, n, tid, Ks, LY::LQ);
        stage_rows<TIn, DV, NTHR>(vr, false, n, tid, Vs, LY::LV);
        if (c0 + CH < t1) {
            kr.load(kh, c0 + CH, min(CH, t1 - c0 - CH), tid);
            vr.load(vh, c0 + CH, min(CH, t1 - c0 - CH), tid);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < CH / M::KB; ++j) {
#pragma unroll
            for (int i = 0; i < LY::RTW; ++i) {
                const typename M::frag a = M::load_tr(Ks, LY::LQ, j * M::KB, 16 * (w * LY::RTW + i), lane);
#pragma unroll
                for (int c = 0; c < LY::NCT; ++c) {
                    const typename M::frag b = (c < DV / 16) ? M::load_tr(Vs, LY::LV, j * M::KB, 16 * c, lane)
                                                             : M::ones();
                    M::mma(acc[i][c], a, b);
                }
            }
        }
        __syncthreads();
    }
}

template <typename TIn, int DK, int DV>
__global__ __launch_bounds__(NTHR) void la_fused_kernel(const TIn* __restrict__ q,
                                                        const TIn* __restrict__ k,
                                                        const TIn* __restrict__ v,
                                                        const float* S0, const float* z0,
                                                        TIn* __restrict__ o, float* S_out, float* z_out,
                                                        int* __restrict__ flags, float* __restrict__ agg,
                                                        float* __restrict__ incl, int T, int L, int G,
                                                        int HT, float eps) {
    using M = Mma<TIn>;
    using op = typename M::op_t;
    using LY = Layout<TIn, DK, DV>;
    constexpr int LQ = LY::LQ, LV = LY::LV, NCT = LY::NCT, RTW = LY::RTW, E = LY::E;
    constexpr int VEC = 16 / sizeof(TIn);
    __shared__ __align__(16) op Qs[CH * LQ];
    __shared__ __align__(16) op Ks[CH * LQ];
    __shared__ __align__(16) op Vs[CH * LV];
    __shared__ __align__(16) op St[(DV + 16) * LQ];
    __shared__ __align__(16) op Os[CH * LV];
    __shared__ int lb_count, lb_timeout;   // look-back result (wave 0 -> block)

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, li = lane & 15;
    const int w = wave_id(tid);
    const int head = blockIdx.x % HT, seg = blockIdx.x / HT;
    const TIn* qh = q + (long)head * T * DK;
    const TIn* kh = k + (long)head * T * DK;
    const TIn* vh = v + (long)head * T * DV;
    TIn* oh = o + (long)head * T * DV;
    const int t_beg = seg * L, t_end = min((seg + 1) * L, T);
    int* hflags = flags + (long)head * G;

    // element of the (dk x (dv + 1)) state held in tile (i, c), register r
    auto row_of = [&](int i, int r) { return 16 * (w * RTW + i) + 4 * g + r; };
    auto state_index = [&](int i, int c, int r) {
        return c < NCT - 1 ? row_of(i, r) * DV + 16 * c + li : DK * DV + row_of(i, r);
    };

    // ---- 1. this segment's aggregate
    v4f A[RTW][NCT];
#pragma unroll
    for (int i = 0; i < RTW; ++i)
#pragma unroll
        for (int c = 0; c < NCT; ++c) A[i][c] = zero4();
    accumulate_kv<TIn, DK, DV>(kh, vh, t_beg, t_end, A, Ks, Vs, tid);

    // ---- 2. publish the aggregate, then walk back for the incoming state
    v4f S[RTW][NCT];
#pragma unroll
    for (int i = 0; i < RTW; ++i)
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int e = state_index(i, c, r);
                float x = 0.f;
                if (c < NCT - 1) { if (S0) x = S0[(long)head * DK * DV + e]; }
                else { if (z0) x = z0[(long)head * DK + (e - DK * DV)]; }
                S[i][c][r] = seg == 0 ? x : 0.f;
            }
    if (seg > 0 && seg + 1 < G) {
        float* dst = agg + ((long)head * G + seg) * E;
#pragma unroll
        for (int i = 0; i < RTW; ++i)
#pragma unroll
            for (int c = 0; c < NCT; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (c < NCT - 1 || li == 0) store_coherent(dst + state_index(i, c, r), A[i][c][r]);
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) store_flag(&hflags[seg], kFlagAggregate);
    }
    if (seg > 0) {
        // Find j*, the nearest predecessor whose inclusive state is published
        // (every segment between j* and this one must have its aggregate
        // out).  Windows of up to 64 predecessors: lane j of wave 0 watches
        // segment base - j.  Segment 0 always publishes an inclusive state,
        // so the walk ends.
        int jstar = -1;
        bool timeout = false;
        for (int base = seg - 1; base >= 0; base -= 64) {
            if (w == 0) {
                const int p = base - lane;
                int polls = 0, found = -1, to = 0;
                while (true) {
                    const int f = p >= 0 ? load_flag(&hflags[p]) : kFlagNone;
                    const unsigned long long incl_mask = __ballot(p >= 0 && f == kFlagInclusive);
                    const unsigned long long ready_mask = __ballot(p < 0 || f != kFlagNone);
                    const int live = __popcll(__ballot(p >= 0));
                    const int stop = incl_mask ? __ffsll((long long)incl_mask) - 1 : 64;
                    const int need = min(stop + 1, live);
                    const unsigned long long need_mask = need >= 64 ? ~0ull : ((1ull << need) - 1);
                    if ((ready_mask & need_mask) == need_mask) {
                        found = incl_mask ? base - stop : -1;
                        break;
                    }
                    if (++polls > kPollLimit) {
                        to = 1;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
                if (lane == 0) {
                    lb_count = found;
                    lb_timeout = to;
                }
            }
            __syncthreads();
            // block-uniform values, made visibly uniform (they guard MFMA loops)
            jstar = __builtin_amdgcn_readfirstlane(lb_count);
            timeout = __builtin_amdgcn_readfirstlane(lb_timeout) != 0;
            __syncthreads();
            if (timeout || jstar >= 0) break;
        }
        if (!timeout) {
            // S_in = incl[j*] + agg[j*+1] + ... + agg[seg-1], left to right: the
            // same rounding as the left-to-right sum from S0, whatever j* is,
            // so results do not depend on timing.
            const float* src = incl + ((long)head * G + jstar) * E;
#pragma unroll
            for (int i = 0; i < RTW; ++i)
#pragma unroll
                for (int c = 0; c < NCT; ++c)
#pragma unroll
                    for (int r = 0; r < 4; ++r) S[i][c][r] = load_coherent(src + state_index(i, c, r));
            for (int p = jstar + 1; p < seg; ++p) {
                const float* a = agg + ((long)head * G + p) * E;
#pragma unroll
                for (int i = 0; i < RTW; ++i)
#pragma unroll
                    for (int c = 0; c < NCT; ++c)
#pragma unroll
                        for (int r = 0; r < 4; ++r) S[i][c][r] += load_coherent(a + state_index(i, c, r));
            }
        } else {
            // recompute the incoming state from the inputs
#pragma unroll
            for (int i = 0; i < RTW; ++i)
#pragma unroll
                for (int c = 0; c < NCT; ++c)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int e = state_index(i, c, r);
                        float x = 0.f;
                        if (c < NCT - 1) { if (S0) x = S0[(long)head * DK * DV + e]; }
                        else { if (z0) x = z0[(long)head * DK + (e - DK * DV)]; }
                        S[i][c][r] = x;
                    }
            accumulate_kv<TIn, DK, DV>(kh, vh, 0, t_beg, S, Ks, Vs, tid);
        }
    }

    // ---- 3. publish the inclusive state (or the final state, last segment)
    if (seg + 1 < G) {
        float* dst = incl + ((long)head * G + seg) * E;
#pragma unroll
        for (int i = 0; i < RTW; ++i)
#pragma unroll
            for (int c = 0; c < NCT; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (c < NCT - 1 || li == 0) store_coherent(dst + state_index(i, c, r), S[i][c][r] + A[i][c][r]);
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) store_flag(&hflags[seg], kFlagInclusive);
    } else {
#pragma unroll
        for (int i = 0; i < RTW; ++i)
#pragma unroll
            for (int c = 0; c < NCT; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int e = state_index(i, c, r);
                    const float x = S[i][c][r] + A[i][c][r];
                    if (c < NCT - 1) { if (S_out) S_out[(long)head * DK * DV + e] = x; }
                    else if (li == 0 && z_out) z_out[(long)head * DK + (e - DK * DV)] = x;
                }
    }

    // ---- 4. the chunk loop from the incoming state
    ChunkRegs<TIn, DK, NTHR> qr, kr;
    ChunkRegs<TIn, DV, NTHR> vr;
    int c0 = t_beg;
    qr.load(qh, c0, min(CH, t_end - c0), tid);
    kr.load(kh, c0, min(CH, t_end - c0), tid);
    vr.load(vh, c0, min(CH, t_end - c0), tid);
    for (; c0 < t_end; c0 += CH) {
        const int n = min(CH, t_end - c0);
        stage_rows<TIn, DK, NTHR>(qr, true, n, tid, Qs, LQ);
        stage_rows<TIn, DK, NTHR>(kr, true, n, tid, Ks, LQ);
        stage_rows<TIn, DV, NTHR>(vr, false, n, tid, Vs, LV);
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            const int rt = w * RTW + i;
#pragma unroll
            for (int c = 0; c < NCT; ++c) {
                op* dst = &St[(16 * c + li) * LQ + 16 * rt + 4 * g];
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[r] = M::cvt(S[i][c][r]);
            }
        }
        if (c0 + CH < t_end) {
            const int n1 = min(CH, t_end - c0 - CH);
            qr.load(qh, c0 + CH, n1, tid);
            kr.load(kh, c0 + CH, n1, tid);
            vr.load(vh, c0 + CH, n1, tid);
        }
        __syncthreads();

        v4f Pt[CH / 16];
#pragma unroll
        for (int kb = 0; kb < CH / 16; ++kb) {
            Pt[kb] = zero4();
            if (kb <= w) {
#pragma unroll
                for (int kk = 0; kk < DK / M::KB; ++kk) {
                    const typename M::frag a = M::load(&Ks[(16 * kb + li) * LQ + kk * M::KB], g);
                    const typename M::frag b = M::load(&Qs[(16 * w + li) * LQ + kk * M::KB], g);
                    M::mma(Pt[kb], a, b);
                }
                if (kb == w) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (4 * g + r > li) Pt[kb][r] = 0.f;
                }
            }
        }
        v4f N[NCT];
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
            N[c] = zero4();
#pragma unroll
            for (int j = 0; j < CH / M::KB; ++j) {
                if (j * M::KB > 16 * w + 15) continue;
                const typename M::frag a = (c < DV / 16) ? M::load_tr(Vs, LV, j * M::KB, 16 * c, lane) : M::ones();
                const typename M::frag b =
                    M::from_tiles(Pt[j * M::KB / 16], Pt[j * M::KB / 16 + (M::KB / 16 - 1)]);
                M::mma(N[c], a, b);
            }
#pragma unroll
            for (int kk = 0; kk < DK / M::KB; ++kk) {
                const typename M::frag a = M::load(&St[(16 * c + li) * LQ + kk * M::KB], g);
                const typename M::frag b = M::load(&Qs[(16 * w + li) * LQ + kk * M::KB], g);
                M::mma(N[c], a, b);
            }
        }
        {
            const float inv = fast_rcp(N[NCT - 1][0] + eps);
#pragma unroll
            for (int c = 0; c < DV / 16; ++c) {
                op* dst = &Os[(16 * w + li) * LV + 16 * c + 4 * g];
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[r] = M::cvt(N[c][r] * inv);
            }
        }
#pragma unroll
        for (int j = 0; j < CH / M::KB; ++j) {
#pragma unroll
            for (int i = 0; i < RTW; ++i) {
                const typename M::frag a = M::load_tr(Ks, LQ, j * M::KB, 16 * (w * RTW + i), lane);
#pragma unroll
                for (int c = 0; c < NCT; ++c) {
                    const typename M::frag b = (c < DV / 16) ? M::load_tr(Vs, LV, j * M::KB, 16 * c, lane)
                                                             : M::ones();
                    M::mma(S[i][c], a, b);
                }
            }
        }
        __syncthreads();
        for (int idx = tid; idx < n * (DV / VEC); idx += NTHR) {
            const int row = idx / (DV / VEC), col = (idx % (DV / VEC)) * VEC;
            *reinterpret_cast<uint4*>(oh + (long)(c0 + row) * DV + col) =
                *reinterpret_cast<const uint4*>(&Os[row * LV + col]);
        }
    }
}

__global__ void la_flags_clear_kernel(int* flags, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) flags[i] = kFlagNone;
}

template <typename TIn, int DK, int DV>
hipError_t launch_typed(const void* q, const void* k, const void* v, const float* S0,
                        const float* z0, void* o, float* S_out, float* z_out, int HT, int T,
                        float eps, const LaPlan& plan, float* ws, hipStream_t stream) {
    const int G = plan.G, L = plan.L;
    int* flags = reinterpret_cast<int*>(ws);
    float* agg = ws + la_flag_words(HT, G);
    float* incl = agg + (size_t)HT * G * (DK * DV + DK);
    la_flags_clear_kernel<<<dim3((HT * G + 255) / 256), dim3(256), 0, stream>>>(flags, HT * G);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    la_fused_kernel<TIn, DK, DV><<<dim3(HT * G), dim3(NTHR), 0, stream>>>(
        static_cast<const TIn*>(q), static_cast<const TIn*>(k), static_cast<const TIn*>(v), S0, z0,
        static_cast<TIn*>(o), S_out, z_out, flags, agg, incl, T, L, G, HT, eps);
    return hipGetLastError();
}

}  // namespace

size_t la_flag_words(int HT, int G) { return ((size_t)HT * G + 63) / 64 * 64; }

LaPlan la_plan(int HT, int T, int dk, int dv) {
    // Enough (head, segment) workgroups for two per compute unit, and segments
    // short enough that the keys and values of all resident workgroups (read
    // twice: aggregate, then outputs) stay within the Infinity Cache.
    const int nch = (T + CH - 1) / CH;
    const long occ = ((long)nch * HT) / 512;
    const long cap = (256L * 1024) / ((long)(dk + dv) * 2 * CH);
    long cps = occ < cap ? occ : cap;
    if (cps < 1) cps = 1;
    LaPlan p;
    p.L = (int)cps * CH;
    p.G = (T + p.L - 1) / p.L;
    return p;
}

size_t la_ws_floats(int HT, int T, int dk, int dv) {
    const LaPlan p = la_plan(HT, T, dk, dv);
    return la_flag_words(HT, p.G) + (size_t)2 * HT * p.G * ((size_t)dk * dv + dk);
}

size_t la_lds_bytes(int dk, int dv, int dtype) {
    const size_t el = dtype == 1 ? 2 : 4;
    const size_t pad = 16 / el;
    return el * ((size_t)2 * CH * (dk + pad) + (size_t)2 * CH * (dv + pad) + (size_t)(dv + 16) * (dk + pad));
}

hipError_t launch_la_forward(const void* q, const void* k, const void* v, const float* S0,
                             const float* z0, void* o, float* S_out, float* z_out, int HT, int T,
                             int dk, int dv, int dtype, float eps, const LaPlan& plan, float* ws,
                             hipStream_t stream) {
#define LA_CASE(TY, DT, A, B)                                                                  \
    if (dtype == DT && dk == A && dv == B)                                                     \
        return launch_typed<TY, A, B>(q, k, v, S0, z0, o, S_out, z_out, HT, T, eps, plan, ws, \
                                      stream);
    LA_CASE(bf16_t, 1, 64, 64)
    LA_CASE(bf16_t, 1, 64, 128)
    LA_CASE(bf16_t, 1, 128, 64)
    LA_CASE(bf16_t, 1, 128, 128)
    LA_CASE(float, 0, 64, 64)
    LA_CASE(float, 0, 64, 128)
    LA_CASE(float, 0, 128, 64)
#undef LA_CASE
    return hipErrorInvalidValue;
}

}  // namespace la
