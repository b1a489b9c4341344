// Chunk-local building blocks of the delta rule used by its backward pass
// (and the per-chunk state tiles that the forward hands to it).
//
// Within a chunk of C = 64 tokens the rule's corrections solve the unit
// lower-triangular system (I + A) U = V - diag(gamma) K S with
//   A[t][i] = (gamma_t / gamma_i) beta_i (k_t . k_i)   (i < t),
// gamma_t the chunk-local product of the forgetting gates up to t (all ones
// for the plain rule: "AIGC 基本功｜线性、循环与记忆架构-LinearMem" §03, the
// corrective write and the decayed variant).  T = (I + A)^{-1} and the
// causal scores P[t][i] = (gamma_t / gamma_i) (q_t . k_i) (i <= t) depend on
// the chunk's own keys, queries, betas and gates only.
#pragma once
#include "common.hpp"

namespace la {
namespace dchunk {

constexpr int CH = kChunk;
constexpr int NT = 512;  // eight waves
constexpr int NWV = 8;
constexpr int LT = CH + 8;  // bf16 rows of C x C matrices
constexpr int LF = CH + 4;  // fp32 rows of the C x C work matrix

// ---------------------------------------------------------------- state tiles
//
// Per-chunk states in HBM (the state entering a chunk, or the gradient of the
// state leaving it), bf16, in MFMA output-fragment order: tile (column tile
// ct, row tile rt) of chunk record ci is 256 consecutive elements, lane l
// holding rows 16 rt + 4 (l / 16) + r, r = 0..3, of column 16 ct + l % 16.
// A wave moves a 16 x 16 tile with one 8-byte access per lane, and two
// vertically adjacent tiles form an MFMA operand with no conversion.
template <int DK, int DV>
__host__ __device__ constexpr long tile_offset(long ci, int ct, int rt, int lane) {
    return ((ci * (DV / 16) + ct) * (DK / 16) + rt) * 256 + (long)lane * 4;
}
__device__ __forceinline__ void put_tile(bf16_t* p, const v4f& x) {
    uint2 pk;
    pk.x = pack_bf16x2(x[0], x[1]);
    pk.y = pack_bf16x2(x[2], x[3]);
    *reinterpret_cast<uint2*>(p) = pk;
}
__device__ __forceinline__ uint2 get_tile(const bf16_t* p) { return *reinterpret_cast<const uint2*>(p); }
// Operand whose contraction rows 0..15 come from tile t0 and 16..31 from t1
// (the slot order of Mma<bf16_t>::from_tiles).
__device__ __forceinline__ v8bf tile_frag(uint2 t0, uint2 t1) {
    return __builtin_bit_cast(v8bf, v4u{t0.x, t0.y, t1.x, t1.y});
}
__device__ __forceinline__ v4f tile_f32(uint2 t) {
    return v4f{__uint_as_float(t.x << 16), __uint_as_float(t.x & 0xffff0000u), __uint_as_float(t.y << 16),
               __uint_as_float(t.y & 0xffff0000u)};
}

// ---------------------------------------------------------------- gates
//
// Wave 0, lane t: the chunk-local cumulative log-gate Gl[t] (each log
// clamped at -20; tokens at or past n count as alpha = 1), Ge[t] = gamma_t =
// exp(Gl[t]) and Gc[t] = gamma_C / gamma_t = exp(Gl[C-1] - Gl[t]).
__device__ __forceinline__ void gate_prefix(float a, int t, int n, float* Gl, float* Ge, float* Gc) {
    float lg = t < n ? fmaxf(logf(a), -20.f) : 0.f;
#pragma unroll
    for (int off = 1; off < CH; off <<= 1) {
        const float y = __shfl_up(lg, off);
        lg += t >= off ? y : 0.f;
    }
    const float lend = __shfl(lg, CH - 1);
    Gl[t] = lg;
    Ge[t] = expf(lg);
    Gc[t] = expf(lend - lg);
}

// The ten lower 16x16 tiles of a 64x64 matrix: diagonal first.
__host__ __device__ constexpr void lower_tile(int id, int& i, int& j) {
    if (id < 4) { i = id; j = id; }
    else if (id < 7) { i = id - 3; j = id - 4; }
    else if (id < 9) { i = id - 5; j = id - 7; }
    else { i = 3; j = 0; }
}

// Zero the six upper 16x16 tiles of a C x C bf16 matrix of layout XL
// (read as zero operands, never written by the builders below).
template <class XL = RowLayout<LT>>
__device__ __forceinline__ void clear_upper(__bf16* X, int tid) {
    for (int e = tid; e < 6 * 256; e += NT) {
        const int tile = e >> 8, r = (e >> 4) & 15, c = e & 15;
        const int bi = tile < 3 ? 0 : tile < 5 ? 1 : 2;
        const int bj = tile < 3 ? tile + 1 : tile < 5 ? tile - 1 : 3;
        X[XL::at(16 * bi + r, 16 * bj + c)] = Mma<bf16_t>::cvt(0.f);
    }
}

// ---------------------------------------------------------------- T and P
//
// Builds T = (I + A)^{-1} (bf16, lower blocks of Ts) and, with WANT_P, the
// causal scores P (bf16, lower blocks of Ps, rows = queries).  Ks, Qs: the
// staged chunk rows (bf16, layout KL: RowLayout; rows past the chunk end
// zero); Bs:
// betas; Gl: cumulative log-gates (GATED).  Af ([C][LF] fp32), Ad and Yf
// (4 x 256 fp32 each) are scratch.  Called by all threads of the workgroup
// after the chunk is staged and visible; ends with a barrier.  With KEEP,
// keep[j] receives the raw K K^T tile (lower tile w + 8 j, j = 0, 1, when
// below 10) that this wave computed for A.
//
// A's diagonal 16x16 blocks are inverted by forward substitution (wave 0,
// one column per lane); the rest by 2x2 block doubling: the inverse of
// [[M11, 0], [M21, M22]] is [[M11^-1, 0], [-M22^-1 M21 M11^-1, M22^-1]],
// first on the 32x32 diagonal blocks, then on the lower-left 32x32 block.
//
// K_DEAD: Af may occupy the same LDS as Ks (K is not needed afterwards):
// every K K^T tile is then computed before the first write of A.
template <int DK, bool GATED, bool WANT_P, bool KEEP = false, class KL = RowLayout<DK + 8>, bool K_DEAD = false>
__device__ __forceinline__ void build_T(const __bf16* Ks, const __bf16* Qs, const float* Bs, const float* Gl,
                                        float* Af, float* Ad, float* Yf, __bf16* Ts, __bf16* Ps, int w, int g,
                                        int li, v4f* keep = nullptr) {
    using M = Mma<bf16_t>;
    using MF = Mma<float>;
    constexpr int NTILE = WANT_P ? 20 : 10;
    if constexpr (K_DEAD) {
        static_assert(!WANT_P && !KEEP, "K_DEAD builds T alone");
        // every one of the ten K K^T tiles must be formed before A overwrites K
        static_assert(2 * NWV >= 10, "K_DEAD needs at least five waves");
        v4f kk[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {  // eight or more waves: at most two of the ten tiles each
            const int id = w + NWV * jj;
            if (id >= 10) break;
            int bi, bj;
            lower_tile(id, bi, bj);
            kk[jj] = zero4();
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb)
                M::mma(kk[jj], KL::frag(Ks, 16 * bi + li, 32 * kb, g), KL::frag(Ks, 16 * bj + li, 32 * kb, g));
        }
        __syncthreads();  // every read of Ks done: its LDS now holds A
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int id = w + NWV * jj;
            if (id >= 10) break;
            int bi, bj;
            lower_tile(id, bi, bj);
            v4f a;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * bi + 4 * g + r, i = 16 * bj + li;
                float x = Bs[i] * kk[jj][r];
                if constexpr (GATED) x *= __expf(Gl[t] - Gl[i]);  // dropped above the diagonal by the select
                a[r] = (i < t) ? x : 0.f;
                Af[t * LF + i] = a[r];
            }
            if (bi == bj) *reinterpret_cast<v4f*>(&Ad[bi * 256 + li * 16 + 4 * g]) = a;
        }
    }
#pragma unroll
    for (int jj = 0; jj < (K_DEAD ? 0 : 3); ++jj) {
        const int id = w + NWV * jj;
        if (id >= NTILE) break;
        int bi, bj;
        lower_tile(id % 10, bi, bj);
        v4f acc = zero4();
        if (id < 10) {
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb)
                M::mma(acc, KL::frag(Ks, 16 * bi + li, 32 * kb, g), KL::frag(Ks, 16 * bj + li, 32 * kb, g));
            if constexpr (KEEP) {
                if (jj < 2) keep[jj] = acc;
            }
            v4f a;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * bi + 4 * g + r, i = 16 * bj + li;
                float x = Bs[i] * acc[r];
                if constexpr (GATED) x *= __expf(Gl[t] - Gl[i]);  // dropped above the diagonal by the select
                a[r] = (i < t) ? x : 0.f;
                Af[t * LF + i] = a[r];
            }
            if (bi == bj) *reinterpret_cast<v4f*>(&Ad[bi * 256 + li * 16 + 4 * g]) = a;
        } else {
            // keys of tile bj (rows) x queries of tile bi (columns): each lane
            // writes four consecutive keys of one query row
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb)
                M::mma(acc, KL::frag(Ks, 16 * bj + li, 32 * kb, g), KL::frag(Qs, 16 * bi + li, 32 * kb, g));
            if constexpr (GATED) {
                const float gq = Gl[16 * bi + li];
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] *= __expf(gq - Gl[16 * bj + 4 * g + r]);
            }
            uint2 pk;
            pk.x = pack_bf16x2((bi == bj && 4 * g + 0 > li) ? 0.f : acc[0], (bi == bj && 4 * g + 1 > li) ? 0.f : acc[1]);
            pk.y = pack_bf16x2((bi == bj && 4 * g + 2 > li) ? 0.f : acc[2], (bi == bj && 4 * g + 3 > li) ? 0.f : acc[3]);
            *reinterpret_cast<uint2*>(&Ps[(16 * bi + li) * LT + 16 * bj + 4 * g]) = pk;
        }
    }
    __syncthreads();
    if (w == 0) {  // diagonal blocks, column-oriented substitution
        const int b = g, j = li;
        float d[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) d[m] = (m == j) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < 15; ++m) {
            const v4f* col = reinterpret_cast<const v4f*>(&Ad[b * 256 + m * 16]);  // A_bb[.][m]
            const v4f c[4] = {col[0], col[1], col[2], col[3]};
#pragma unroll
            for (int i = m + 1; i < 16; ++i) d[i] -= c[i >> 2][i & 3] * d[m];
        }
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            Af[(16 * b + m) * LF + 16 * b + j] = d[m];
            Ts[(16 * b + m) * LT + 16 * b + j] = M::cvt(d[m]);
        }
    }
    __syncthreads();
    auto rowA = [&](int r0, int c0) { return *reinterpret_cast<const v4f*>(&Af[(r0 + li) * LF + c0 + 4 * g]); };
    auto colB = [&](int r0, int c0) {
        v4f bb;
#pragma unroll
        for (int s = 0; s < 4; ++s) bb[s] = Af[(r0 + 4 * g + s) * LF + c0 + li];
        return bb;
    };
    auto yB = [&](int t) {
        v4f bb;
#pragma unroll
        for (int s = 0; s < 4; ++s) bb[s] = Yf[t * 256 + (4 * g + s) * 16 + li];
        return bb;
    };
    auto put_T = [&](int bi, int bj, const v4f& x) {
#pragma unroll
        for (int r = 0; r < 4; ++r) Ts[(16 * bi + 4 * g + r) * LT + 16 * bj + li] = M::cvt(x[r]);
    };
    if (w == 1 || w == 2) {  // T10 = -D1 A10 D0 (wave 1), T32 = -D3 A32 D2 (wave 2)
        const int lo = w == 1 ? 0 : 32;
        v4f P = zero4(), X = zero4();
        MF::mma(P, rowA(lo + 16, lo), colB(lo, lo));
        MF::mma(X, rowA(lo + 16, lo + 16), P);
        X = -X;
#pragma unroll
        for (int r = 0; r < 4; ++r) Af[(lo + 4 * g + r) * LF + lo + 16 + li] = X[r];  // kept in the unused upper block
        put_T(lo / 16 + 1, lo / 16, X);
    }
    __syncthreads();
    if (w >= 1 && w <= 4) {  // Y = A_BL T_TL
        const int t = w - 1, yr = t >> 1, yc = t & 1;
        v4f Y = zero4();
        if (yc == 0) {
            MF::mma(Y, rowA(32 + 16 * yr, 0), colB(0, 0));
            MF::mma(Y, rowA(32 + 16 * yr, 16), colB(0, 16));
        } else {
            MF::mma(Y, rowA(32 + 16 * yr, 16), colB(16, 16));
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) Yf[t * 256 + (4 * g + r) * 16 + li] = Y[r];
    }
    __syncthreads();
    if (w >= 1 && w <= 4) {  // T_BL = -T_BR Y
        const int t = w - 1, xr = t >> 1, xc = t & 1;
        v4f X = zero4();
        if (xr == 0) {
            MF::mma(X, rowA(32, 32), yB(xc));
        } else {
            MF::mma(X, rowA(32, 48), yB(xc));
            MF::mma(X, rowA(48, 48), yB(2 + xc));
        }
        put_T(2 + xr, xc, -X);
    }
    __syncthreads();
}

// The causal scores P (bf16, lower blocks of Ps, rows = queries; gated: o
// Gamma) alone, for loops that load T from the chunk records; wave w builds
// lower tiles w and w + 8.  With KEEP, keep[j] receives the raw K K^T tile
// w + 8 j (j = 0, 1, when below 10).  KL, QL, PL: the LDS layouts of K, Q
// and P (RowLayout).  No barrier.
template <int DK, bool GATED, bool KEEP = false, class KL = RowLayout<DK + 8>, class QL = KL,
          class PL = RowLayout<LT>>
__device__ __forceinline__ void build_P(const __bf16* Ks, const __bf16* Qs, const float* Gl, __bf16* Ps, int w, int g,
                                        int li, v4f* keep = nullptr) {
    using M = Mma<bf16_t>;
    static_assert(2 * NWV >= 10, "two tiles per wave must cover the ten lower tiles");
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int id = w + NWV * jj;
        if (id >= 10) break;
        int bi, bj;
        lower_tile(id, bi, bj);
        v4f acc = zero4();
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb)
            M::mma(acc, KL::frag(Ks, 16 * bj + li, 32 * kb, g), QL::frag(Qs, 16 * bi + li, 32 * kb, g));
        if constexpr (GATED) {
            const float gq = Gl[16 * bi + li];
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] *= __expf(gq - Gl[16 * bj + 4 * g + r]);
        }
        uint2 pk;
        pk.x = pack_bf16x2((bi == bj && 4 * g + 0 > li) ? 0.f : acc[0], (bi == bj && 4 * g + 1 > li) ? 0.f : acc[1]);
        pk.y = pack_bf16x2((bi == bj && 4 * g + 2 > li) ? 0.f : acc[2], (bi == bj && 4 * g + 3 > li) ? 0.f : acc[3]);
        *reinterpret_cast<uint2*>(&Ps[PL::at(16 * bi + li, 16 * bj + 4 * g)]) = pk;
        if constexpr (KEEP) {
            v4f kk = zero4();
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb)
                M::mma(kk, KL::frag(Ks, 16 * bi + li, 32 * kb, g), KL::frag(Ks, 16 * bj + li, 32 * kb, g));
            keep[jj] = kk;
        }
    }
}

// A chunk record: the ten lower 16 x 16 tiles of a lower block-triangular
// 64 x 64 bf16 matrix (the upper tiles are zero and not stored), in
// lower_tile order, each tile's rows of 16 contiguous: 320 pieces of 16
// bytes (5 KB instead of 8).  Piece p holds row 16 bi + (p / 2) % 16,
// columns 16 bj + 8 (p % 2) .. + 7 of tile p / 32.  Readers clear the upper
// tiles of their LDS copy once (clear_upper) and stage only these pieces.
constexpr int kRecTiles = 10;
constexpr int kRecElems = kRecTiles * 256;
constexpr int kRecPieces = kRecElems / 8;
__device__ __forceinline__ void rec_piece(int p, int& row, int& col) {
    int bi, bj;
    lower_tile(p >> 5, bi, bj);
    row = 16 * bi + ((p >> 1) & 15);
    col = 16 * bj + 8 * (p & 1);
}
// this thread's piece of a record (threads kRecPieces.. hold none)
__device__ __forceinline__ uint4 load_rec(const bf16_t* rec, int tid) {
    return tid < kRecPieces ? *reinterpret_cast<const uint4*>(rec + tid * 8) : make_uint4(0u, 0u, 0u, 0u);
}
// the piece into LDS rows of layout XL (natural or group-permuted)
template <class XL = RowLayout<LT>>
__device__ __forceinline__ void stage_rec(__bf16* Xs, uint4 x, int tid) {
    if (tid >= kRecPieces) return;
    int r, c;
    rec_piece(tid, r, c);
    __bf16* row = &Xs[r * XL::LD];
    if constexpr (XL::PERM) {
        *reinterpret_cast<uint2*>(row + pcol(c)) = make_uint2(x.x, x.y);
        *reinterpret_cast<uint2*>(row + pcol(c + 4)) = make_uint2(x.z, x.w);
    } else {
        *reinterpret_cast<uint4*>(row + c) = x;
    }
}

}  // namespace dchunk
}  // namespace la
