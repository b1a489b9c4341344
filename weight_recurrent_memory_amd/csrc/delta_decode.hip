// Delta-rule fast-weight memory, single-token decode step on a resident fp32
// state, updated in place ("AIGC 基本功｜线性、循环与记忆架构-LinearMem" §03
// "从累加改成纠错" and "手撕：递推与记忆模型" "Delta-rule fast weight" for the
// write; §05 of the first page for the in-place inference update):
//   u = v - S^T k,   S <- S + beta k u^T,   o = S^T q   (write, then read).
//
// Like the linear-attention decode step this is a streaming read-modify-write
// of S (dk*dv floats per state, one workgroup per (sequence, head) state), but
// the write needs S^T k over the whole old state first.  Thread t owns four
// consecutive value columns (one 16-byte vector) of every R-th state row and
// keeps them in registers: it folds its rows into partial S^T k and S^T q,
// the partials meet in LDS, each thread sums the ones of its columns, and
// then updates its registers and streams them back.  The read uses the old
// state: o = S^T q + beta u (k . q).
//
// Gated form (LinearMem §03, the Gated DeltaNet rule): the old state is first
// decayed by alpha, S~ = alpha S, and the step above runs on S~.  Here alpha
// scales the two reductions and the state as it is written back.
//
// Scalar-decay form ("线性注意力与 SSM" §3, Mamba-2): S <- alpha S + k v^T,
// o = S^T q = alpha S^T q + (k . q) v: no correction, so S^T k is not needed.
//
// Serving input transforms (flags; LinearMem §05, §08): kNormQK scales q and
// k to unit L2 norm (applied as factors on the reductions and the write),
// kBetaSigmoid reads beta as a logit.  pred (optional) receives the
// prediction (decayed S)^T k made before the write.
#include "common.hpp"
#include "kernels.hpp"

namespace la {

namespace {

constexpr int NTHR = 256;

enum : int { kRuleDelta = 0, kRuleGatedDelta = 1, kRuleSsd = 2 };

// NORM (the q/k L2 normalisation) is a template parameter: as a runtime
// option it costs the kernel about 60 registers and half its occupancy.
template <typename TIn, int DK, int DV, int RULE, bool NORM>
__global__ __launch_bounds__(NTHR) void delta_decode_kernel(const TIn* __restrict__ q,
                                                            const TIn* __restrict__ k,
                                                            const TIn* __restrict__ v,
                                                            const TIn* __restrict__ beta,
                                                            const float* __restrict__ alpha,
                                                            float* __restrict__ S, TIn* __restrict__ o,
                                                            TIn* __restrict__ pred_out, int flags) {
    constexpr int CG = DV / 4;    // 16-byte column groups per row
    constexpr int R = NTHR / CG;  // row groups
    constexpr int RPT = DK / R;   // rows per thread
    static_assert(RPT * R == DK && CG * 4 == DV && DK <= NTHR, "shape");
    __shared__ float fk[DK], fq[DK];
    __shared__ v4f part_k[R][CG], part_q[R][CG];
    __shared__ float kq_part[NTHR / 64], kk_part[NTHR / 64], qq_part[NTHR / 64];

    constexpr bool GATED = RULE != kRuleDelta, SSD = RULE == kRuleSsd;
    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;
    const long s = blockIdx.x;
    float* Ss = S + s * DK * DV;

    // the state loads first: they do not depend on q, k, v
    v4f st[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        st[m] = *reinterpret_cast<const v4f*>(Ss + (long)(rg + R * m) * DV + 4 * cg);

    float kq = 0.f, kk = 0.f, qq = 0.f;
    if (tid < DK) {
        const float kv = Elem<TIn>::load(k, s * DK + tid);
        const float qv = Elem<TIn>::load(q, s * DK + tid);
        fk[tid] = kv;
        fq[tid] = qv;
        kq = kv * qv;
        kk = kv * kv;
        qq = qv * qv;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        kq += __shfl_xor(kq, off);
        if constexpr (NORM) {
            kk += __shfl_xor(kk, off);
            qq += __shfl_xor(qq, off);
        }
    }
    if ((tid & 63) == 0) {
        kq_part[tid >> 6] = kq;
        if constexpr (NORM) {
            kk_part[tid >> 6] = kk;
            qq_part[tid >> 6] = qq;
        }
    }
    const float braw = SSD ? 1.f : Elem<TIn>::load(beta, s);
    const float b = (!SSD && (flags & kBetaSigmoid)) ? 1.f / (1.f + __expf(-braw)) : braw;
    const float a = GATED ? alpha[s] : 1.f;
    const v4f vv = v4f{Elem<TIn>::load(v, s * DV + 4 * cg + 0), Elem<TIn>::load(v, s * DV + 4 * cg + 1),
                       Elem<TIn>::load(v, s * DV + 4 * cg + 2), Elem<TIn>::load(v, s * DV + 4 * cg + 3)};
    __syncthreads();

    // partial S^T k and S^T q over this thread's rows
    v4f pk = zero4(), pq = zero4();
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int row = rg + R * m;
        if constexpr (!SSD) pk += fk[row] * st[m];
        pq += fq[row] * st[m];
    }
    if constexpr (!SSD) part_k[rg][cg] = pk;
    part_q[rg][cg] = pq;
    __syncthreads();

    // every thread sums the partials of its own columns (broadcast reads)
    v4f pred = zero4(), sq = zero4();
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if constexpr (!SSD) pred += part_k[r][cg];
        sq += part_q[r][cg];
    }
    // unit-norm factors of k and q (1 without the transform; a zero row stays zero)
    float rk = 1.f, rq = 1.f;
    if constexpr (NORM) {
        float ks = 0.f, qs = 0.f;
#pragma unroll
        for (int i = 0; i < NTHR / 64; ++i) {
            ks += kk_part[i];
            qs += qq_part[i];
        }
        rk = ks > 0.f ? __builtin_amdgcn_rsqf(ks) : 0.f;
        rq = qs > 0.f ? __builtin_amdgcn_rsqf(qs) : 0.f;
    }
    pred *= (GATED ? a : 1.f) * rk;  // reductions over the decayed state
    sq *= (GATED ? a : 1.f) * rq;
    const v4f u = vv - pred;
    const v4f bu = b * u;

    // write: S += beta k u^T, streamed back (the state set does not fit the
    // Infinity Cache, so keeping its lines there would only cost write-backs)
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int row = rg + R * m;
        const v4f x = (GATED ? a * st[m] : st[m]) + (fk[row] * rk) * bu;
        __builtin_nontemporal_store(x, reinterpret_cast<v4f*>(Ss + (long)row * DV + 4 * cg));
    }

    // read with the updated state: o = S^T q + beta u (k . q)
    if (rg == 0) {
        float kqs = 0.f;
#pragma unroll
        for (int i = 0; i < NTHR / 64; ++i) kqs += kq_part[i];
        const v4f out = sq + (kqs * rk * rq) * bu;
#pragma unroll
        for (int e = 0; e < 4; ++e) Elem<TIn>::store(o, s * DV + 4 * cg + e, out[e]);
        if (!SSD && pred_out) {
#pragma unroll
            for (int e = 0; e < 4; ++e) Elem<TIn>::store(pred_out, s * DV + 4 * cg + e, pred[e]);
        }
    }
}

template <typename TIn, int DK, int DV, int RULE, bool NORM>
void launch_one(const void* q, const void* k, const void* v, const void* beta, const float* alpha, float* S,
                void* o, void* pred, int flags, int NH, hipStream_t stream) {
    delta_decode_kernel<TIn, DK, DV, RULE, NORM><<<dim3(NH), dim3(NTHR), 0, stream>>>(
        static_cast<const TIn*>(q), static_cast<const TIn*>(k), static_cast<const TIn*>(v),
        static_cast<const TIn*>(beta), alpha, S, static_cast<TIn*>(o), static_cast<TIn*>(pred), flags);
}

template <typename TIn, int DK, int DV, int RULE>
void launch_rule(const void* q, const void* k, const void* v, const void* beta, const float* alpha, float* S,
                 void* o, void* pred, int flags, int NH, hipStream_t stream) {
    if (flags & kNormQK)
        launch_one<TIn, DK, DV, RULE, true>(q, k, v, beta, alpha, S, o, pred, flags, NH, stream);
    else
        launch_one<TIn, DK, DV, RULE, false>(q, k, v, beta, alpha, S, o, pred, flags, NH, stream);
}

// beta NULL (with alpha) selects the scalar-decay rule; alpha NULL the plain delta rule.
template <typename TIn, int DK, int DV>
hipError_t launch_typed(const void* q, const void* k, const void* v, const void* beta, const float* alpha,
                        float* S, void* o, void* pred, int flags, int NH, hipStream_t stream) {
    if (!alpha)
        launch_rule<TIn, DK, DV, kRuleDelta>(q, k, v, beta, nullptr, S, o, pred, flags, NH, stream);
    else if (beta)
        launch_rule<TIn, DK, DV, kRuleGatedDelta>(q, k, v, beta, alpha, S, o, pred, flags, NH, stream);
    else
        launch_one<TIn, DK, DV, kRuleSsd, false>(q, k, v, nullptr, alpha, S, o, nullptr, 0, NH, stream);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_delta_decode(const void* q, const void* k, const void* v, const void* beta,
                               const float* alpha, float* S, void* o, void* pred, int flags, int NH, int dk,
                               int dv, int dtype, hipStream_t stream) {
#define DEC_CASE(TY, DT, A, B)             \
    if (dtype == DT && dk == A && dv == B) \
        return launch_typed<TY, A, B>(q, k, v, beta, alpha, S, o, pred, flags, NH, stream);
    DEC_CASE(bf16_t, 1, 64, 64)
    DEC_CASE(bf16_t, 1, 64, 128)
    DEC_CASE(bf16_t, 1, 128, 64)
    DEC_CASE(bf16_t, 1, 128, 128)
    DEC_CASE(float, 0, 64, 64)
    DEC_CASE(float, 0, 64, 128)
    DEC_CASE(float, 0, 128, 64)
    DEC_CASE(float, 0, 128, 128)
#undef DEC_CASE
    return hipErrorInvalidValue;
}

}  // namespace la
