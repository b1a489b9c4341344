// Causal ELU+1 linear attention, single-token decode step on a resident
// fp32 state, updated in place ("AIGC 基本功｜线性、循环与记忆架构-LinearMem"
// §03 for the recurrence and read-out, §05 for the in-place inference update):
//   S <- S + phi(k) v^T,  z <- z + phi(k),  o = phi(q)^T S / (phi(q)^T z + eps).
//
// The step is a streaming read-modify-write of S (dk*dv floats per state,
// written back with non-temporal stores):
// one workgroup per (sequence, head) state.  Thread t owns four consecutive
// value columns (one 16-byte vector) of every R-th state row, so each wave
// reads and writes whole 512-byte (dv = 128) or 256-byte (dv = 64) rows.  The
// updated row is folded into phi(q)^T S on the fly from registers; the
// partial sums over rows meet in LDS.  The denominator uses z updated by the
// first dk threads.
#include "common.hpp"
#include "kernels.hpp"

namespace la {

namespace {

constexpr int NTHR = 256;

template <typename TIn, int DK, int DV>
__global__ __launch_bounds__(NTHR) void la_decode_kernel(const TIn* __restrict__ q,
                                                         const TIn* __restrict__ k,
                                                         const TIn* __restrict__ v,
                                                         float* __restrict__ S,
                                                         float* __restrict__ z,
                                                         TIn* __restrict__ o, float eps) {
    constexpr int CG = DV / 4;         // 16-byte column groups per row
    constexpr int R = NTHR / CG;       // row groups
    constexpr int RPT = DK / R;        // rows per thread
    static_assert(RPT * R == DK && CG * 4 == DV, "shape");
    __shared__ float fq[DK], fk[DK];
    __shared__ v4f part[R][CG];
    __shared__ float den_part[NTHR / 64];

    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;
    const long s = blockIdx.x;
    float* Ss = S + s * DK * DV;

    // Issue the state loads first: they do not depend on q, k, v.
    v4f st[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        st[m] = *reinterpret_cast<const v4f*>(Ss + (long)(rg + R * m) * DV + 4 * cg);

    float dpart = 0.f;
    if (tid < DK) {
        const float fkv = phi(Elem<TIn>::load(k, s * DK + tid));
        const float fqv = phi(Elem<TIn>::load(q, s * DK + tid));
        fk[tid] = fkv;
        fq[tid] = fqv;
        const float zn = z[s * DK + tid] + fkv;
        z[s * DK + tid] = zn;
        dpart = fqv * zn;
    }
    const v4f vv = v4f{Elem<TIn>::load(v, s * DV + 4 * cg + 0), Elem<TIn>::load(v, s * DV + 4 * cg + 1),
                       Elem<TIn>::load(v, s * DV + 4 * cg + 2), Elem<TIn>::load(v, s * DV + 4 * cg + 3)};
    // wave reduction of the denominator parts
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dpart += __shfl_xor(dpart, off);
    if ((tid & 63) == 0) den_part[tid >> 6] = dpart;
    __syncthreads();

    v4f acc = zero4();
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int row = rg + R * m;
        const float f = fk[row];
        v4f x = st[m] + f * vv;
        // streaming store: a 1 GB state set does not fit the Infinity Cache, so
        // keeping the written lines there only costs write-backs later
        __builtin_nontemporal_store(x, reinterpret_cast<v4f*>(Ss + (long)row * DV + 4 * cg));
        acc += fq[row] * x;
    }
    part[rg][cg] = acc;
    __syncthreads();

    if (tid < DV) {
        float num = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) num += part[r][tid >> 2][tid & 3];
        float den = eps;
#pragma unroll
        for (int i = 0; i < NTHR / 64; ++i) den += den_part[i];
        Elem<TIn>::store(o, s * DV + tid, num / den);
    }
}

template <typename TIn, int DK, int DV>
hipError_t launch_typed(const void* q, const void* k, const void* v, float* S, float* z, void* o,
                        int NH, float eps, hipStream_t stream) {
    la_decode_kernel<TIn, DK, DV><<<dim3(NH), dim3(NTHR), 0, stream>>>(
        static_cast<const TIn*>(q), static_cast<const TIn*>(k), static_cast<const TIn*>(v), S, z,
        static_cast<TIn*>(o), eps);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_la_decode(const void* q, const void* k, const void* v, float* S, float* z,
                            void* o, int NH, int dk, int dv, int dtype, float eps,
                            hipStream_t stream) {
#define DEC_CASE(TY, DT, A, B) \
    if (dtype == DT && dk == A && dv == B) return launch_typed<TY, A, B>(q, k, v, S, z, o, NH, eps, stream);
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
