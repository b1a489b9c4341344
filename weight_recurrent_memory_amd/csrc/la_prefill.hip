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
// Sequence parallelism: each head's tokens are cut into G segments.  Because
// the state update is additive, the state entering segment g is
// S0 + sum_{g' < g} (segment sum of g').  Three launches:
//   la_segsum   one workgroup per (head, segment): phi(K)^T [V | 1] over it
//   la_segscan  exclusive prefix over segments (in place), final state out
//   la_segout   one workgroup per (head, segment): the chunk loop above
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
    static constexpr int LQ = DK + PAD;          // rows indexed by token (or dv), k = dk
    static constexpr int LT = CH + PAD;          // rows indexed by dk (or dv), k = token
    static constexpr int NCT = DV / 16 + 1;      // value column tiles + the ones/z tile
    static constexpr int RTW = DK / 64;          // dk row tiles per wave (4 waves)
    static constexpr int E = DK * DV + DK;       // floats per (head, segment) state
};

// ------------------------------------------------------------- la_segsum

template <typename TIn, int DK, int DV>
__global__ __launch_bounds__(NTHR) void la_segsum_kernel(const TIn* __restrict__ k,
                                                         const TIn* __restrict__ v,
                                                         float* __restrict__ ws, int T, int L, int G) {
    using M = Mma<TIn>;
    using op = typename M::op_t;
    using LY = Layout<TIn, DK, DV>;
    __shared__ __align__(16) op Kt[DK * LY::LT];
    __shared__ __align__(16) op Vt[DV * LY::LT];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, li = lane & 15;
    const int head = blockIdx.x / G, seg = blockIdx.x % G;
    const TIn* kh = k + (long)head * T * DK;
    const TIn* vh = v + (long)head * T * DV;

    v4f acc[LY::RTW][LY::NCT];
#pragma unroll
    for (int i = 0; i < LY::RTW; ++i)
#pragma unroll
        for (int c = 0; c < LY::NCT; ++c) acc[i][c] = zero4();

    const int t_end = min((seg + 1) * L, T);
    for (int c0 = seg * L; c0 < t_end; c0 += CH) {
        const int n = min(CH, t_end - c0);
        ChunkRegs<TIn, DK, NTHR> kr;
        ChunkRegs<TIn, DV, NTHR> vr;
        kr.load(kh, c0, n, tid);
        vr.load(vh, c0, n, tid);
        stage<TIn, DK, NTHR, false, true>(kr, true, n, tid, nullptr, 0, Kt, LY::LT);
        stage<TIn, DV, NTHR, false, true>(vr, false, n, tid, nullptr, 0, Vt, LY::LT);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < LY::RTW; ++i) {
            const int rt = w * LY::RTW + i;
#pragma unroll
            for (int j = 0; j < CH / M::KB; ++j) {
                const typename M::frag a = M::load(&Kt[(16 * rt + li) * LY::LT + j * M::KB], g);
#pragma unroll
                for (int c = 0; c < LY::NCT; ++c) {
                    const typename M::frag b = (c < DV / 16)
                        ? M::load(&Vt[(16 * c + li) * LY::LT + j * M::KB], g) : M::ones();
                    M::mma(acc[i][c], a, b);
                }
            }
        }
        __syncthreads();
    }

    float* out = ws + (long)(head * G + seg) * LY::E;
#pragma unroll
    for (int i = 0; i < LY::RTW; ++i) {
        const int rt = w * LY::RTW + i;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * rt + 4 * g + r;
#pragma unroll
            for (int c = 0; c < DV / 16; ++c) out[row * DV + 16 * c + li] = acc[i][c][r];
            if (li == 0) out[DK * DV + row] = acc[i][LY::NCT - 1][r];
        }
    }
}

// ------------------------------------------------------------ la_segscan

// One thread per state element; serial over the G segments of its head.
__global__ __launch_bounds__(256) void la_segscan_kernel(float* __restrict__ ws, const float* S0,
                                                         const float* z0, float* S_out, float* z_out,
                                                         int G, int dk, int dv) {
    const int E = dk * dv + dk;
    const int head = blockIdx.y;
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= E) return;
    float acc = 0.f;
    if (e < dk * dv) {
        if (S0) acc = S0[(long)head * dk * dv + e];
    } else {
        if (z0) acc = z0[(long)head * dk + (e - dk * dv)];
    }
    float* p = ws + (long)head * G * E + e;
    for (int s = 0; s < G; ++s) {
        const float x = p[(long)s * E];
        p[(long)s * E] = acc;
        acc += x;
    }
    if (e < dk * dv) {
        if (S_out) S_out[(long)head * dk * dv + e] = acc;
    } else {
        if (z_out) z_out[(long)head * dk + (e - dk * dv)] = acc;
    }
}

// ------------------------------------------------------------- la_segout

template <typename TIn, int DK, int DV>
__global__ __launch_bounds__(NTHR) void la_segout_kernel(const TIn* __restrict__ q,
                                                         const TIn* __restrict__ k,
                                                         const TIn* __restrict__ v,
                                                         TIn* __restrict__ o,
                                                         const float* __restrict__ ws,
                                                         int T, int L, int G, float eps) {
    using M = Mma<TIn>;
    using op = typename M::op_t;
    using LY = Layout<TIn, DK, DV>;
    constexpr int LQ = LY::LQ, LT = LY::LT, NCT = LY::NCT;
    __shared__ __align__(16) op Qs[CH * LQ];          // phi(Q_c), k = dk
    __shared__ __align__(16) op Ks[CH * LQ];          // phi(K_c), k = dk
    __shared__ __align__(16) op Kt[DK * LT];          // phi(K_c)^T, k = token
    __shared__ __align__(16) op Vt[DV * LT];          // V_c^T, k = token
    __shared__ __align__(16) op St[(DV + 16) * LQ];   // [S | z..z]^T, k = dk

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, li = lane & 15;
    const int head = blockIdx.x / G, seg = blockIdx.x % G;
    const TIn* qh = q + (long)head * T * DK;
    const TIn* kh = k + (long)head * T * DK;
    const TIn* vh = v + (long)head * T * DV;
    TIn* oh = o + (long)head * T * DV;

    // State entering this segment, in output-tile layout: wave w owns dk rows
    // [16*RTW*w, 16*RTW*(w+1)); the last column tile holds z in every column.
    v4f S[LY::RTW][NCT];
    {
        const float* st = ws + (long)(head * G + seg) * LY::E;
#pragma unroll
        for (int i = 0; i < LY::RTW; ++i) {
            const int rt = w * LY::RTW + i;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * rt + 4 * g + r;
#pragma unroll
                for (int c = 0; c < DV / 16; ++c) S[i][c][r] = st[row * DV + 16 * c + li];
                S[i][NCT - 1][r] = st[DK * DV + row];
            }
        }
    }

    const int t_end = min((seg + 1) * L, T);
    for (int c0 = seg * L; c0 < t_end; c0 += CH) {
        const int n = min(CH, t_end - c0);
        {
            ChunkRegs<TIn, DK, NTHR> qr, kr;
            ChunkRegs<TIn, DV, NTHR> vr;
            qr.load(qh, c0, n, tid);
            kr.load(kh, c0, n, tid);
            vr.load(vh, c0, n, tid);
            stage<TIn, DK, NTHR, true, false>(qr, true, n, tid, Qs, LQ, nullptr, 0);
            stage<TIn, DK, NTHR, true, true>(kr, true, n, tid, Ks, LQ, Kt, LT);
            stage<TIn, DV, NTHR, false, true>(vr, false, n, tid, nullptr, 0, Vt, LT);
        }
        // state before this chunk -> St (transposed, operand precision)
#pragma unroll
        for (int i = 0; i < LY::RTW; ++i) {
            const int rt = w * LY::RTW + i;
#pragma unroll
            for (int c = 0; c < NCT; ++c) {
                op* dst = &St[(16 * c + li) * LQ + 16 * rt + 4 * g];
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[r] = M::cvt(S[i][c][r]);
            }
        }
        __syncthreads();

        // P^T tiles for this wave's 16 queries: Pt[kb] holds keys 16kb..16kb+15.
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
                        if (4 * g + r > li) Pt[kb][r] = 0.f;  // key after query: masked
                }
            }
        }

        // num / den for this wave's queries, one column tile at a time.
        v4f N[NCT];
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
            N[c] = zero4();
#pragma unroll
            for (int j = 0; j < CH / M::KB; ++j) {
                if (j * M::KB > 16 * w + 15) continue;  // keys entirely after the queries
                const typename M::frag a = M::from_tiles(Pt[j * M::KB / 16], Pt[j * M::KB / 16 + (M::KB / 16 - 1)]);
                const typename M::frag b = (c < DV / 16)
                    ? M::load(&Vt[(16 * c + li) * LT + j * M::KB], g) : M::ones();
                M::mma(N[c], a, b);
            }
#pragma unroll
            for (int kk = 0; kk < DK / M::KB; ++kk) {
                const typename M::frag a = M::load(&Qs[(16 * w + li) * LQ + kk * M::KB], g);
                const typename M::frag b = M::load(&St[(16 * c + li) * LQ + kk * M::KB], g);
                M::mma(N[c], a, b);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * w + 4 * g + r;
            if (row < n) {
                const float inv = 1.f / (N[NCT - 1][r] + eps);
#pragma unroll
                for (int c = 0; c < DV / 16; ++c)
                    Elem<TIn>::store(oh, (long)(c0 + row) * DV + 16 * c + li, N[c][r] * inv);
            }
        }

        // S += phi(K_c)^T [V_c | 1]
#pragma unroll
        for (int i = 0; i < LY::RTW; ++i) {
            const int rt = w * LY::RTW + i;
#pragma unroll
            for (int j = 0; j < CH / M::KB; ++j) {
                const typename M::frag a = M::load(&Kt[(16 * rt + li) * LT + j * M::KB], g);
#pragma unroll
                for (int c = 0; c < NCT; ++c) {
                    const typename M::frag b = (c < DV / 16)
                        ? M::load(&Vt[(16 * c + li) * LT + j * M::KB], g) : M::ones();
                    M::mma(S[i][c], a, b);
                }
            }
        }
        __syncthreads();
    }
}

template <typename TIn, int DK, int DV>
hipError_t launch_typed(const void* q, const void* k, const void* v, const float* S0,
                        const float* z0, void* o, float* S_out, float* z_out, int HT, int T,
                        float eps, const LaPlan& plan, float* ws, hipStream_t stream) {
    const int G = plan.G, L = plan.L;
    la_segsum_kernel<TIn, DK, DV><<<dim3(HT * G), dim3(NTHR), 0, stream>>>(
        static_cast<const TIn*>(k), static_cast<const TIn*>(v), ws, T, L, G);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int E = DK * DV + DK;
    la_segscan_kernel<<<dim3((E + 255) / 256, HT), dim3(256), 0, stream>>>(ws, S0, z0, S_out, z_out,
                                                                           G, DK, DV);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    la_segout_kernel<TIn, DK, DV><<<dim3(HT * G), dim3(NTHR), 0, stream>>>(
        static_cast<const TIn*>(q), static_cast<const TIn*>(k), static_cast<const TIn*>(v),
        static_cast<TIn*>(o), ws, T, L, G, eps);
    return hipGetLastError();
}

}  // namespace

size_t la_lds_bytes(int dk, int dv, int dtype) {
    const size_t el = dtype == 1 ? 2 : 4;
    const size_t pad = 16 / el;
    return el * ((size_t)2 * CH * (dk + pad) + (size_t)dk * (CH + pad) + (size_t)dv * (CH + pad) +
                 (size_t)(dv + 16) * (dk + pad));
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
