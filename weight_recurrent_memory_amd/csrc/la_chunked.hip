// Causal ELU+1 linear attention prefill blocked into chunks of C = 16, 32 or
// 128 tokens, for uniform batches.
//
// The function is the one of la_prefill.hip ("AIGC 基本功｜线性、循环与记忆
// 架构-LinearMem" §03: S_t = S_{t-1} + phi(k_t) v_t^T, z_t = z_{t-1} +
// phi(k_t), o_t = phi(q_t)^T S_t / (phi(q_t)^T z_t + eps), write then
// read); only the blocking differs.  The chunked form -- a small masked
// attention inside each chunk plus the state carried across chunks ("线性
// 注意力与 SSM:两条技术路线的完整推导" §3, Mamba-2 paragraph; "手撕：递推与
// 记忆模型", "Chunked scan", where a scan handed its state every few tokens
// equals one pass) -- gives the same outputs for every chunk size up to
// rounding, which is what this path lets callers check on the device: per
// chunk of C tokens entered with state [S | z],
//   P = tril(phi(Q) phi(K)^T)                      (C x C, keys after a query zero)
//   N^T = [V | 1]^T P^T + [S | z]^T phi(Q)^T        (numerators and denominators)
//   o = N / (den + eps),  [S | z] += phi(K)^T [V | 1].
// The fused 64-token kernel splits the state by rows and shares it through
// LDS; here each wave (four for dv = 64, eight for dv = 128) owns whole
// value-column tiles of [S | z] (fp32, registers), so its own tiles are the
// A operand of its outputs and only the chunk's phi(K), V, phi(Q) and P go
// through LDS.  The z tile's owner forms the denominators, which the others
// read after a barrier.
//
// Sequence parallelism as in la_backward.hip: segment sums, their prefix,
// then every segment's chunk loop from its entering state (three launches).
#include "common.hpp"
#include "kernels.hpp"
#include "la_chunked.hpp"

namespace la {

namespace {

template <typename TIn, int DK, int DV, int C>
struct CL {
    // waves: four for dv = 64, eight for dv = 128 (five or nine column tiles;
    // at most two per wave)
    static constexpr int NW = DV == 128 ? 8 : 4;
    static constexpr int NT = 64 * NW;
    using M = Mma<TIn>;
    using op = typename M::op_t;
    static constexpr int KB = M::KB;                  // contraction per fragment: 32 (bf16), 16 (fp32)
    static constexpr int CP = C < KB ? KB : C;        // rows staged: the chunk zero-padded to whole fragments
    static constexpr int PAD = 16 / (int)sizeof(op);  // 16 bytes of padding per row
    static constexpr int LQ = DK + PAD;               // rows of phi(Q), phi(K)
    static constexpr int LV = DV + PAD;               // rows of V
    static constexpr int LP = CP + PAD;               // rows of P (one per query, keys along the row)
    static constexpr int NVT = DV / 16;               // value column tiles
    static constexpr int NCT = NVT + 1;               // and the z tile (16 equal columns)
    static constexpr int XR = DK / 16;                // dk row tiles of a state column tile
    static constexpr int NQT = C / 16;                // query (and key) tiles of a chunk
    static constexpr int SLOTS = (NCT + NW - 1) / NW; // state column tiles per wave: tiles w, w + NW, ...
    static constexpr int KT = KB / 16;                // output tiles per fragment's contraction
    static constexpr int E = DK * DV + DK;            // floats of one [S | z] state, S row-major, then z
    static constexpr int KS = CP * LQ, QS = CP * LQ, VS = CP * LV, PS = C * LP;
    static constexpr int BYTES = (int)sizeof(op) * (KS + QS + VS + PS) + C * 4;  // + 1 / (den + eps)
    static_assert(C % 16 == 0 && CP % KB == 0, "chunk of whole 16-row tiles");
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// Rows [c0, c0 + CP) of one (sequence, head)'s [T][D] input into LDS rows of
// stride ld, phi applied when PHI; rows at or past n (the chunk's rows
// inside the segment, n <= C) are zero after the feature map, so padded and
// out-of-range keys add nothing.
template <typename TIn, int D, int CP, bool PHI, int NT>
__device__ __forceinline__ void stage_chunk(const TIn* head, int c0, int n, typename Mma<TIn>::op_t* dst, int ld,
                                            int tid) {
    using M = Mma<TIn>;
    using op = typename M::op_t;
    constexpr int VEC = 16 / (int)sizeof(TIn);
    static_assert(sizeof(op) == sizeof(TIn), "operands keep the input width");
    for (int e = tid; e < CP * D / VEC; e += NT) {
        const int row = e / (D / VEC), col = (e % (D / VEC)) * VEC;
        op vals[VEC];
        if (row < n) {
            TIn raw[VEC];
            *reinterpret_cast<uint4*>(raw) = *reinterpret_cast<const uint4*>(head + (long)(c0 + row) * D + col);
#pragma unroll
            for (int u = 0; u < VEC; ++u) {
                const float x = Elem<TIn>::load(raw, u);
                vals[u] = M::cvt(PHI ? phi(x) : x);
            }
        } else {
#pragma unroll
            for (int u = 0; u < VEC; ++u) vals[u] = M::cvt(0.f);
        }
        *reinterpret_cast<uint4*>(dst + row * ld + col) = *reinterpret_cast<const uint4*>(vals);
    }
}

// Four consecutive operands from four floats.
template <typename op>
__device__ __forceinline__ void put4(op* p, const v4f& x) {
    if constexpr (sizeof(op) == 2) {
        *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
    } else {
        *reinterpret_cast<v4f*>(p) = x;
    }
}

enum { kSum = 0, kOut = 1 };

// One workgroup per (sequence, head, segment).  kSum: segments 0..G-2, the
// segment's phi(K)^T [V | 1] from zero into agg.  kOut: every segment from
// its entering state in state_in, writing o, and S_out, z_out after the
// last segment of each sequence.
template <typename TIn, int DK, int DV, int C, int MODE>
__global__ __launch_bounds__(DV == 128 ? 512 : 256) void la_chunk_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const float* __restrict__ state_in, float* __restrict__ agg, TIn* __restrict__ o, float* __restrict__ S_out,
    float* __restrict__ z_out, float eps, SegMap sm) {
    using Y = CL<TIn, DK, DV, C>;
    using M = Mma<TIn>;
    using op = typename M::op_t;
    using frag = typename M::frag;
    constexpr bool OUT = MODE == kOut;
    constexpr int KB = Y::KB, LQ = Y::LQ, LV = Y::LV, LP = Y::LP, KT = Y::KT, XR = Y::XR, NQT = Y::NQT;
    constexpr int NVT = Y::NVT, NCT = Y::NCT, SLOTS = Y::SLOTS, CP = Y::CP, NW = Y::NW, NT = Y::NT;
    static_assert(NT == (DV == 128 ? 512 : 256), "launch bounds");
    __shared__ __align__(16) unsigned char smem[Y::BYTES];
    op* Ks = reinterpret_cast<op*>(smem);
    op* Qs = Ks + Y::KS;
    op* Vs = Qs + Y::QS;
    op* Ps = Vs + Y::VS;
    float* Rd = reinterpret_cast<float*>(Ps + Y::PS);  // 1 / (den + eps) per query of the chunk

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, li = lane & 15;
    const int w = wave_id(tid);
    __builtin_assume(w >= 0 && w < NW);
    const int G1 = OUT ? sm.G : sm.G - 1;
    const int vh = blockIdx.x / G1, seg = blockIdx.x % G1;  // vh = sequence * H + head
    const long slot = (long)vh * sm.G + seg;
    const long row0 = (long)vh * sm.T;  // the (sequence, head)'s first input row
    const int t0 = seg * sm.L, t_end = min(t0 + sm.L, sm.T);
    const TIn* qh = q + row0 * DK;
    const TIn* kh = k + row0 * DK;
    const TIn* vhp = v + row0 * DV;

    // this wave's column tiles of [S | z]: X[j][i] = rows 16 i + 4 g + r,
    // column 16 id + li of tile id = w + NW j (the z tile's columns all equal z)
    v4f X[SLOTS][XR];
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
        const int id = w + NW * j;
#pragma unroll
        for (int i = 0; i < XR; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * i + 4 * g + r;
                float x = 0.f;
                if (OUT && id < NCT) {
                    const float* st = state_in + slot * Y::E;
                    x = id < NVT ? st[row * DV + 16 * id + li] : st[DK * DV + row];
                }
                X[j][i][r] = x;
            }
    }
    if constexpr (OUT) {  // P's upper tiles and padding columns are read as zeros and never written
        for (int e = tid; e < Y::PS; e += NT) Ps[e] = M::cvt(0.f);
    }

    for (int c0 = t0; c0 < t_end; c0 += C) {
        const int n = min(C, t_end - c0);
        stage_chunk<TIn, DK, CP, true, NT>(kh, c0, n, Ks, LQ, tid);
        stage_chunk<TIn, DV, CP, false, NT>(vhp, c0, n, Vs, LV, tid);
        if constexpr (OUT) stage_chunk<TIn, DK, CP, true, NT>(qh, c0, n, Qs, LQ, tid);
        __syncthreads();

        if constexpr (OUT) {
            // P as transposed tiles (keys of tile bj x queries of tile bi):
            // each lane holds four consecutive keys of one query row
            for (int t = w; t < NQT * (NQT + 1) / 2; t += NW) {
                int bi = 0, rem = t;
                while (rem > bi) rem -= ++bi;  // t = bi (bi + 1) / 2 + bj, bj <= bi
                const int bj = rem;
                v4f acc = zero4();
#pragma unroll
                for (int kk = 0; kk < DK / KB; ++kk)
                    M::mma(acc, M::load(&Ks[(16 * bj + li) * LQ + KB * kk], g), M::load(&Qs[(16 * bi + li) * LQ + KB * kk], g));
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (bi == bj && 4 * g + r > li) acc[r] = 0.f;
                put4(&Ps[(16 * bi + li) * LP + 16 * bj + 4 * g], acc);
            }
            __syncthreads();
            // denominators 1^T P^T + z^T phi(Q)^T from the z tile's owner
#pragma unroll
            for (int j = 0; j < SLOTS; ++j) {
                if (w + NW * j != NVT) continue;
                for (int qt = 0; qt < NQT; ++qt) {
                    v4f d = zero4();
#pragma unroll
                    for (int kb = 0; kb < CP / KB; ++kb) {
                        if (KB * kb > 16 * qt + 15) continue;  // keys after every query of the tile
                        M::mma(d, M::ones(), M::load(&Ps[(16 * qt + li) * LP + KB * kb], g));
                    }
#pragma unroll
                    for (int kk = 0; kk < DK / KB; ++kk)
                        M::mma(d, M::from_tiles(X[j][KT * kk], X[j][KT * kk + KT - 1]),
                               M::load(&Qs[(16 * qt + li) * LQ + KB * kk], g));
                    if (g == 0) Rd[16 * qt + li] = 1.f / (d[0] + eps);
                }
            }
            __syncthreads();
            // numerators of this wave's value tiles, normalised and stored
#pragma unroll
            for (int j = 0; j < SLOTS; ++j) {
                const int id = w + NW * j;
                if (id >= NVT) continue;
                for (int qt = 0; qt < NQT; ++qt) {
                    v4f nt = zero4();
#pragma unroll
                    for (int kb = 0; kb < CP / KB; ++kb) {
                        if (KB * kb > 16 * qt + 15) continue;
                        M::mma(nt, M::load_tr(Vs, LV, KB * kb, 16 * id, lane), M::load(&Ps[(16 * qt + li) * LP + KB * kb], g));
                    }
#pragma unroll
                    for (int kk = 0; kk < DK / KB; ++kk)
                        M::mma(nt, M::from_tiles(X[j][KT * kk], X[j][KT * kk + KT - 1]),
                               M::load(&Qs[(16 * qt + li) * LQ + KB * kk], g));
                    const int t = 16 * qt + li;  // query; the lane holds value columns 16 id + 4 g ..
                    if (t < n) {
                        const v4f y = nt * Rd[t];
                        TIn* dst = o + (row0 + c0 + t) * DV + 16 * id + 4 * g;
                        if constexpr (sizeof(TIn) == 2) {
                            *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
                        } else {
                            *reinterpret_cast<v4f*>(dst) = y;
                        }
                    }
                }
            }
        }
        // [S | z] += phi(K)^T [V | 1] on this wave's tiles
#pragma unroll
        for (int j = 0; j < SLOTS; ++j) {
            const int id = w + NW * j;
            if (id >= NCT) continue;
#pragma unroll
            for (int kb = 0; kb < CP / KB; ++kb) {
                const frag vb = id < NVT ? M::load_tr(Vs, LV, KB * kb, 16 * id, lane) : M::ones();
#pragma unroll
                for (int i = 0; i < XR; ++i) M::mma(X[j][i], M::load_tr(Ks, LQ, KB * kb, 16 * i, lane), vb);
            }
        }
        __syncthreads();  // every read of this chunk's LDS rows done
    }

    // the segment's result: its sum (kSum), or the sequence's final state
    float* dS;
    float* dz;
    if constexpr (OUT) {
        if (seg != sm.G - 1) return;
        dS = S_out ? S_out + (long)vh * DK * DV : nullptr;
        dz = z_out ? z_out + (long)vh * DK : nullptr;
    } else {
        dS = agg + slot * Y::E;
        dz = dS + DK * DV;
    }
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
        const int id = w + NW * j;
        if (id >= NCT) continue;
#pragma unroll
        for (int i = 0; i < XR; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * i + 4 * g + r;
                if (id < NVT) {
                    if (dS) dS[row * DV + 16 * id + li] = X[j][i][r];
                } else if (dz && li == 0) {
                    dz[row] = X[j][i][r];
                }
            }
    }
}

// state_in of segment g = [S0 | z0] (or zero) + the sums of segments 0..g-1;
// one thread per element of one (sequence, head)'s state.
__global__ __launch_bounds__(256) void la_chunk_prefix_kernel(const float* __restrict__ agg, const float* S0,
                                                              const float* z0, float* __restrict__ state_in, int HT,
                                                              int G, int dk, int dv) {
    const long E = (long)dk * dv + dk;
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long)HT * E) return;
    const long vh = idx / E, e = idx % E;
    float x = 0.f;
    if (e < (long)dk * dv) {
        if (S0) x = S0[vh * dk * dv + e];
    } else if (z0) {
        x = z0[vh * dk + (e - (long)dk * dv)];
    }
    const long base = vh * G;
    for (int s = 0; s < G; ++s) {
        state_in[(base + s) * E + e] = x;
        if (s + 1 < G) x += agg[(base + s) * E + e];
    }
}

template <typename TIn, int DK, int DV, int C>
hipError_t launch_typed(const TIn* q, const TIn* k, const TIn* v, const float* S0, const float* z0, TIn* o,
                        float* S_out, float* z_out, const SegMap& sm, float eps, float* ws, hipStream_t stream) {
    using Y = CL<TIn, DK, DV, C>;
    const long HT = (long)sm.N * sm.H;
    float* agg = ws;
    float* state_in = ws + HT * sm.G * Y::E;
    hipError_t err;
    if (sm.G > 1) {
        la_chunk_kernel<TIn, DK, DV, C, kSum><<<dim3((unsigned)(HT * (sm.G - 1))), dim3(Y::NT), 0, stream>>>(
            q, k, v, nullptr, agg, nullptr, nullptr, nullptr, eps, sm);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    const long total = HT * Y::E;
    la_chunk_prefix_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream>>>(agg, S0, z0, state_in,
                                                                                         (int)HT, sm.G, DK, DV);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    la_chunk_kernel<TIn, DK, DV, C, kOut><<<dim3((unsigned)(HT * sm.G)), dim3(Y::NT), 0, stream>>>(
        q, k, v, state_in, nullptr, o, S_out, z_out, eps, sm);
    return hipGetLastError();
}

template <typename TIn, int C>
hipError_t launch_dims(const void* q, const void* k, const void* v, const float* S0, const float* z0, void* o,
                       float* S_out, float* z_out, const SegMap& sm, int dk, int dv, float eps, float* ws,
                       hipStream_t stream) {
    const TIn* qt = static_cast<const TIn*>(q);
    const TIn* kt = static_cast<const TIn*>(k);
    const TIn* vt = static_cast<const TIn*>(v);
    TIn* ot = static_cast<TIn*>(o);
#define LAC_CASE(A, B)                                                                                   \
    if (dk == A && dv == B)                                                                              \
        return launch_typed<TIn, A, B, C>(qt, kt, vt, S0, z0, ot, S_out, z_out, sm, eps, ws, stream);
    LAC_CASE(64, 64)
    LAC_CASE(64, 128)
    LAC_CASE(128, 64)
    LAC_CASE(128, 128)
#undef LAC_CASE
    return hipErrorInvalidValue;
}

}  // namespace

bool la_chunked_supported(int chunk, int dtype) {
    if (dtype == 1) return chunk == 16 || chunk == 32 || chunk == 128;
    if (dtype == 0) return chunk == 16 || chunk == 32;
    return false;
}

size_t la_chunked_ws_floats(long slots, int dk, int dv) { return 2 * (size_t)slots * ((size_t)dk * dv + dk); }

hipError_t launch_la_forward_chunked(const void* q, const void* k, const void* v, const float* S0,
                                     const float* z0, void* o, float* S_out, float* z_out, const SegMap& sm,
                                     int dk, int dv, int dtype, float eps, int chunk, float* ws,
                                     hipStream_t stream) {
    if (sm.packed() || !la_chunked_supported(chunk, dtype) || sm.L % chunk != 0) return hipErrorInvalidValue;
    if (dtype == 1) {
        if (chunk == 16) return launch_dims<bf16_t, 16>(q, k, v, S0, z0, o, S_out, z_out, sm, dk, dv, eps, ws, stream);
        if (chunk == 32) return launch_dims<bf16_t, 32>(q, k, v, S0, z0, o, S_out, z_out, sm, dk, dv, eps, ws, stream);
        return launch_dims<bf16_t, 128>(q, k, v, S0, z0, o, S_out, z_out, sm, dk, dv, eps, ws, stream);
    }
    if (chunk == 16) return launch_dims<float, 16>(q, k, v, S0, z0, o, S_out, z_out, sm, dk, dv, eps, ws, stream);
    return launch_dims<float, 32>(q, k, v, S0, z0, o, S_out, z_out, sm, dk, dv, eps, ws, stream);
}

}  // namespace la
