// Delta-rule prefill blocked into chunks of C = 16, 32 or 128 tokens
// (ungated, bf16 inputs, uniform batches).
//
// The rule ("AIGC 基本功｜线性、循环与记忆架构-LinearMem" §03, the corrective
// write; "手撕：递推与记忆模型", "Delta-rule fast weight"):
// S_t = S_{t-1} + beta_t k_t (v_t - S_{t-1}^T k_t)^T, o_t = S_t^T q_t.  Over a
// chunk entered with state S, the corrections u_t = v_t - S_{t-1}^T k_t solve
//   (I + A) U = V - K S,   A[t][i] = beta_i (k_t . k_i) for i < t (else 0),
// and then O = Q S + P (beta o U) with P = tril(Q K^T) (diagonal included)
// and S' = S + K^T (beta o U).  delta_prefill.hip does this for 64-token
// chunks with T = (I + A)^{-1} built by a parallel pass; here the chunk is
// C tokens and the system is solved inside the loop by blocked forward
// substitution over its 16-token tiles: U_b = T_bb (R_b - sum_{c<b} A_bc U_c)
// with T_bb = (I + A_bb)^{-1} of each 16 x 16 diagonal block (fp32
// substitution, one column per lane).  The result equals the sequential
// rule for every C up to rounding ("Chunked scan" of the Recurrence page).
//
// Each of the eight waves owns whole column tiles of the state (fp32,
// registers) and carries its corrections, outputs and state update; the
// chunk's K, V, Q, A (then P, in the same buffer) and the diagonal
// inverses are shared through LDS.  Sequence parallelism as in
// delta_prefill.hip: segment maps (M_g, N_g) by the same loop started from
// (I, 0) without outputs, their composition, then every segment's loop.
#include "common.hpp"
#include "kernels.hpp"
#include "la_chunked.hpp"

namespace la {

namespace {

constexpr int NWD = 8;          // waves
constexpr int NTD = 64 * NWD;   // threads

enum { kMapMode = 0, kOutMode = 1 };

template <int DK, int DV, int C, int MODE>
struct DCL {
    static constexpr bool MAP = MODE == kMapMode;
    static constexpr int KB = 32;                 // bf16 contraction per fragment
    static constexpr int CP = C < KB ? KB : C;    // rows staged: the chunk zero-padded to whole fragments
    static constexpr int LQ = DK + 8, LV = DV + 8;
    static constexpr int LP = CP + 8;             // rows of A (then P): tokens of the chunk along the row
    static constexpr int LTB = KB + 8;            // rows of a diagonal inverse: 16 tokens, 16 zeros, padding
    static constexpr int NQT = C / 16;            // 16-token tiles of a chunk
    static constexpr int NCN = DV / 16;           // state (or N) column tiles
    static constexpr int NCT = MAP ? NCN + DK / 16 : NCN;  // MAP: and the M column tiles
    static constexpr int SLOTS = (NCT + NWD - 1) / NWD;    // column tiles per wave: w, w + 8
    static constexpr int XR = DK / 16;
    static constexpr int KS = CP * LQ, QS = MAP ? 0 : CP * LQ, VS = CP * LV, XS = C * LP, TBS = NQT * 16 * LTB;
    static constexpr int BYTES = 2 * (KS + QS + VS + XS + TBS) + 4 * (NQT * 256 + C);  // + fp32 diagonal A, beta
    static_assert(C % 16 == 0, "chunk of whole 16-token tiles");
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// Rows [c0, c0 + CP) of one (sequence, head)'s [T][D] bf16 input into LDS;
// rows at or past n are zero.
template <int D, int CP>
__device__ __forceinline__ void stage_rows_to(const bf16_t* head, int c0, int n, __bf16* dst, int ld, int tid) {
    for (int e = tid; e < CP * D / 8; e += NTD) {
        const int row = e / (D / 8), col = (e % (D / 8)) * 8;
        uint4 x = make_uint4(0u, 0u, 0u, 0u);
        if (row < n) x = *reinterpret_cast<const uint4*>(head + (long)(c0 + row) * D + col);
        *reinterpret_cast<uint4*>(dst + row * ld + col) = x;
    }
}

// One workgroup per (sequence, head, segment).  kMapMode: segments 0..G-2,
// the segment's map from (M, N) = (I, 0) into map_m, map_n.  kOutMode:
// every segment from its entering state in state_in, writing o, and S_out
// after the last segment of each sequence.
template <int DK, int DV, int C, int MODE>
__global__ __launch_bounds__(NTD) void delta_chunked_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ beta, const float* __restrict__ state_in, float* __restrict__ map_n,
    float* __restrict__ map_m, bf16_t* __restrict__ o, float* __restrict__ S_out, SegMap sm) {
    using Y = DCL<DK, DV, C, MODE>;
    using M = Mma<bf16_t>;
    using frag = M::frag;
    constexpr bool MAP = Y::MAP;
    constexpr int LQ = Y::LQ, LV = Y::LV, LP = Y::LP, LTB = Y::LTB, NQT = Y::NQT, XR = Y::XR, CP = Y::CP;
    constexpr int NCN = Y::NCN, NCT = Y::NCT, SLOTS = Y::SLOTS;
    __shared__ __align__(16) unsigned char smem[Y::BYTES];
    __bf16* Ks = reinterpret_cast<__bf16*>(smem);
    __bf16* Qs = Ks + Y::KS;
    __bf16* Vs = Qs + Y::QS;
    __bf16* Xs = Vs + Y::VS;   // A (bf16, strictly lower), then P
    __bf16* Tb = Xs + Y::XS;   // diagonal inverses T_bb: rows 16 b + m, columns 0..15 (16..31 zero)
    float* Ad = reinterpret_cast<float*>(Tb + Y::TBS);  // fp32 diagonal blocks of A
    float* Bs = Ad + NQT * 256;                          // beta

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, li = lane & 15;
    const int w = wave_id(tid);
    __builtin_assume(w >= 0 && w < NWD);
    const int G1 = MAP ? sm.G - 1 : sm.G;
    const int vh = blockIdx.x / G1, seg = blockIdx.x % G1;  // vh = sequence * H + head
    const long slot = (long)vh * sm.G + seg;
    const long row0 = (long)vh * sm.T;
    const int t0 = seg * sm.L, t_end = min(t0 + sm.L, sm.T);

    // this wave's column tiles: X[j][i] = rows 16 i + 4 g + r, column 16 c + li
    // of tile id = w + 8 j; ids below NCN are S (or N) columns, the rest M's
    v4f X[SLOTS][XR];
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
        const int id = w + NWD * j;
#pragma unroll
        for (int i = 0; i < XR; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * i + 4 * g + r;
                float x = 0.f;
                if (id < NCT) {
                    if constexpr (MAP) x = (id >= NCN && row == 16 * (id - NCN) + li) ? 1.f : 0.f;
                    else x = state_in[slot * DK * DV + row * DV + 16 * id + li];
                }
                X[j][i][r] = x;
            }
    }
    // never written below: A's (and P's) upper tiles and padding columns,
    // the inverses' zero half
    for (int e = tid; e < Y::XS; e += NTD) Xs[e] = M::cvt(0.f);
    for (int e = tid; e < Y::TBS; e += NTD) Tb[e] = M::cvt(0.f);

    for (int c0 = t0; c0 < t_end; c0 += C) {
        const int n = min(C, t_end - c0);
        stage_rows_to<DK, CP>(k + row0 * DK, c0, n, Ks, LQ, tid);
        stage_rows_to<DV, CP>(v + row0 * DV, c0, n, Vs, LV, tid);
        if constexpr (!MAP) stage_rows_to<DK, CP>(q + row0 * DK, c0, n, Qs, LQ, tid);
        for (int t = tid; t < C; t += NTD) Bs[t] = t < n ? bf16_to_f32(beta[row0 + c0 + t]) : 0.f;
        __syncthreads();

        // A's lower tiles (t in tile bi, i in tile bj <= bi); the diagonal
        // blocks also in fp32
        for (int t = w; t < NQT * (NQT + 1) / 2; t += NWD) {
            int bi = 0, rem = t;
            while (rem > bi) rem -= ++bi;  // t = bi (bi + 1) / 2 + bj
            const int bj = rem;
            v4f acc = zero4();
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk)
                M::mma(acc, M::load(&Ks[(16 * bi + li) * LQ + 32 * kk], g), M::load(&Ks[(16 * bj + li) * LQ + 32 * kk], g));
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tt = 16 * bi + 4 * g + r, ii = 16 * bj + li;
                const float a = ii < tt ? Bs[ii] * acc[r] : 0.f;
                Xs[tt * LP + ii] = M::cvt(a);
                if (bi == bj) Ad[bi * 256 + (4 * g + r) * 16 + li] = a;
            }
        }
        __syncthreads();
        // T_bb = (I + A_bb)^{-1}: column li of block b by forward substitution
        for (int e = tid; e < C; e += NTD) {
            const int b = e >> 4, j = e & 15;
            float d[16];
#pragma unroll
            for (int m = 0; m < 16; ++m) d[m] = m == j ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < 15; ++m)
#pragma unroll
                for (int i = m + 1; i < 16; ++i) d[i] -= Ad[b * 256 + i * 16 + m] * d[m];
#pragma unroll
            for (int m = 0; m < 16; ++m) Tb[(16 * b + m) * LTB + j] = M::cvt(d[m]);
        }
        __syncthreads();

        // corrections of column tile j: R = V - K S, then
        // U_b = T_bb (R_b - sum_{c < b} A_bc U_c), and beta o U
        auto solve = [&](int j, v4f (&U)[NQT]) {
            const int id = w + NWD * j;
#pragma unroll
            for (int tt = 0; tt < NQT; ++tt) {
                v4f ks = zero4();
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk)
                    M::mma(ks, M::load(&Ks[(16 * tt + li) * LQ + 32 * kk], g), M::from_tiles(X[j][2 * kk], X[j][2 * kk + 1]));
                v4f acc;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * tt + 4 * g + r;
                    acc[r] = (id < NCN ? (float)Vs[t * LV + 16 * id + li] : 0.f) - ks[r];
                }
                v4f sub = zero4();
#pragma unroll
                for (int c = 0; c < tt; c += 2)
                    M::mma(sub, M::load(&Xs[(16 * tt + li) * LP + 16 * c], g),
                           M::from_tiles(U[c], c + 1 < tt ? U[c + 1] : zero4()));
                acc -= sub;
                U[tt] = zero4();
                M::mma(U[tt], M::load(&Tb[(16 * tt + li) * LTB], g), M::from_tiles(acc, zero4()));
            }
#pragma unroll
            for (int tt = 0; tt < NQT; ++tt)
#pragma unroll
                for (int r = 0; r < 4; ++r) U[tt][r] *= Bs[16 * tt + 4 * g + r];
        };
        // S += K^T (beta o U) on column tile j
        auto update = [&](int j, const v4f (&U)[NQT]) {
#pragma unroll
            for (int kb = 0; kb < CP / 32; ++kb) {
                const frag ub = M::from_tiles(2 * kb < NQT ? U[2 * kb] : zero4(), 2 * kb + 1 < NQT ? U[2 * kb + 1] : zero4());
#pragma unroll
                for (int i = 0; i < XR; ++i) M::mma(X[j][i], M::load_tr(Ks, LQ, 32 * kb, 16 * i, lane), ub);
            }
        };

        if constexpr (MAP) {  // no outputs: each tile's corrections go straight into its state
#pragma unroll
            for (int j = 0; j < SLOTS; ++j) {
                if (w + NWD * j >= NCT) continue;
                v4f U[NQT];
                solve(j, U);
                update(j, U);
                __builtin_amdgcn_sched_barrier(0);  // one tile at a time: its corrections die here
            }
        } else {
            v4f U[SLOTS][NQT];
#pragma unroll
            for (int j = 0; j < SLOTS; ++j)
                if (w + NWD * j < NCT) solve(j, U[j]);
            __syncthreads();  // every read of A done: P takes its buffer
            for (int t = w; t < NQT * (NQT + 1) / 2; t += NWD) {
                int bi = 0, rem = t;
                while (rem > bi) rem -= ++bi;
                const int bj = rem;
                v4f acc = zero4();
#pragma unroll
                for (int kk = 0; kk < DK / 32; ++kk)
                    M::mma(acc, M::load(&Ks[(16 * bj + li) * LQ + 32 * kk], g), M::load(&Qs[(16 * bi + li) * LQ + 32 * kk], g));
                // transposed tile: four consecutive keys 16 bj + 4 g .. of query 16 bi + li
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (bi == bj && 4 * g + r > li) acc[r] = 0.f;
                *reinterpret_cast<uint2*>(&Xs[(16 * bi + li) * LP + 16 * bj + 4 * g]) =
                    make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
            }
            __syncthreads();
            // outputs O^T = S^T Q^T + (beta o U)^T P^T of this wave's columns,
            // from the state entering the chunk, then the state update
#pragma unroll
            for (int j = 0; j < SLOTS; ++j) {
                const int id = w + NWD * j;
                if (id >= NCN) continue;
                for (int qt = 0; qt < NQT; ++qt) {
                    v4f ot = zero4();
#pragma unroll
                    for (int kk = 0; kk < DK / 32; ++kk)
                        M::mma(ot, M::from_tiles(X[j][2 * kk], X[j][2 * kk + 1]), M::load(&Qs[(16 * qt + li) * LQ + 32 * kk], g));
#pragma unroll
                    for (int kb = 0; kb < CP / 32; ++kb) {
                        if (32 * kb > 16 * qt + 15) continue;  // keys after every query of the tile
                        M::mma(ot, M::from_tiles(2 * kb < NQT ? U[j][2 * kb] : zero4(), 2 * kb + 1 < NQT ? U[j][2 * kb + 1] : zero4()),
                               M::load(&Xs[(16 * qt + li) * LP + 32 * kb], g));
                    }
                    const int t = 16 * qt + li;
                    if (t < n)
                        *reinterpret_cast<uint2*>(o + (row0 + c0 + t) * DV + 16 * id + 4 * g) =
                            make_uint2(pack_bf16x2(ot[0], ot[1]), pack_bf16x2(ot[2], ot[3]));
                }
                update(j, U[j]);
            }
        }
        __syncthreads();  // every read of this chunk's LDS rows done
    }

    // the segment's maps, or the sequence's final state
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
        const int id = w + NWD * j;
        if (id >= NCT) continue;
        float* dst;
        int ld, col;
        if constexpr (MAP) {
            const bool is_m = id >= NCN;
            dst = is_m ? map_m + slot * DK * DK : map_n + slot * DK * DV;
            ld = is_m ? DK : DV;
            col = 16 * (is_m ? id - NCN : id) + li;
        } else {
            if (seg != sm.G - 1 || !S_out) return;
            dst = S_out + (long)vh * DK * DV;
            ld = DV;
            col = 16 * id + li;
        }
#pragma unroll
        for (int i = 0; i < XR; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(16 * i + 4 * g + r) * ld + col] = X[j][i][r];
    }
}

template <int DK, int DV, int C>
hipError_t launch_typed(const bf16_t* q, const bf16_t* k, const bf16_t* v, const bf16_t* beta, const float* S0,
                        bf16_t* o, float* S_out, const SegMap& sm, float* ws, hipStream_t stream) {
    const long slots = (long)sm.N * sm.H * sm.G;
    float* map_n = ws;
    float* map_m = map_n + slots * DK * DV;
    float* state_in = map_m + slots * DK * DK;
    const unsigned HT = (unsigned)(sm.N * sm.H);
    hipError_t err;
    if (sm.G > 1) {
        delta_chunked_kernel<DK, DV, C, kMapMode><<<dim3(HT * (sm.G - 1)), dim3(NTD), 0, stream>>>(
            q, k, v, beta, nullptr, map_n, map_m, nullptr, nullptr, sm);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if ((err = launch_delta_compose(map_n, map_m, S0, state_in, sm, DK, DV, stream)) != hipSuccess) return err;
    delta_chunked_kernel<DK, DV, C, kOutMode><<<dim3(HT * sm.G), dim3(NTD), 0, stream>>>(
        q, k, v, beta, state_in, nullptr, nullptr, o, S_out, sm);
    return hipGetLastError();
}

template <int C>
hipError_t launch_dims(const bf16_t* q, const bf16_t* k, const bf16_t* v, const bf16_t* beta, const float* S0,
                       bf16_t* o, float* S_out, const SegMap& sm, int dk, int dv, float* ws, hipStream_t stream) {
#define DCH_CASE(A, B) \
    if (dk == A && dv == B) return launch_typed<A, B, C>(q, k, v, beta, S0, o, S_out, sm, ws, stream);
    DCH_CASE(64, 64)
    DCH_CASE(64, 128)
    DCH_CASE(128, 64)
    DCH_CASE(128, 128)
#undef DCH_CASE
    return hipErrorInvalidValue;
}

}  // namespace

bool delta_chunked_supported(int chunk) { return chunk == 16 || chunk == 32 || chunk == 128; }

size_t delta_chunked_ws_floats(long slots, int dk, int dv) {
    // per slot: N_g, M_g, S_in
    return (size_t)slots * (2 * (size_t)dk * dv + (size_t)dk * dk);
}

hipError_t launch_delta_forward_chunked(const void* q, const void* k, const void* v, const void* beta,
                                        const float* S0, void* o, float* S_out, const SegMap& sm, int dk, int dv,
                                        int chunk, float* ws, hipStream_t stream) {
    if (sm.packed() || !delta_chunked_supported(chunk) || sm.L % chunk != 0) return hipErrorInvalidValue;
    const bf16_t* qb = static_cast<const bf16_t*>(q);
    const bf16_t* kb = static_cast<const bf16_t*>(k);
    const bf16_t* vb = static_cast<const bf16_t*>(v);
    const bf16_t* bb = static_cast<const bf16_t*>(beta);
    bf16_t* ob = static_cast<bf16_t*>(o);
    if (chunk == 16) return launch_dims<16>(qb, kb, vb, bb, S0, ob, S_out, sm, dk, dv, ws, stream);
    if (chunk == 32) return launch_dims<32>(qb, kb, vb, bb, S0, ob, S_out, sm, dk, dv, ws, stream);
    return launch_dims<128>(qb, kb, vb, bb, S0, ob, S_out, sm, dk, dv, ws, stream);
}

}  // namespace la
