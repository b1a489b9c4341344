// Backward pass of the delta rule and of its gated form on gfx950: the
// gradients of L = sum_t dO_t . o_t + <dS_T, S_T> with respect to q, k, v,
// beta, alpha (gated) and S_0, recomputing the forward states.
//
// The rule ("AIGC 基本功｜线性、循环与记忆架构-LinearMem" §03, the corrective
// write and its decayed variant; "手撕：递推与记忆模型", "Delta-rule fast
// weight"): S_t = alpha_t S_{t-1} + beta_t k_t (v_t - alpha_t S_{t-1}^T k_t)^T,
// o_t = S_t^T q_t.  The page's remedy for training memory (§03: split the
// sequence into chunks, keep only chunk-boundary states, recompute inside) is
// the plan here.
//
// Chunk form (C = 64 tokens, state S entering the chunk, gamma the
// chunk-local gate products, Gamma[t][i] = gamma_t / gamma_i, Gc = gamma_C /
// gamma, T = (I + A)^{-1} as in delta_chunk.hpp, P = tril(Q K^T) o Gamma):
//   R = V - diag(gamma) K S,   U = T R,   Ub = diag(beta) U,
//   O = diag(gamma) Q S + P Ub,   S' = gamma_C S + K^T diag(Gc) Ub.
// Given G' = dL/dS' and the chunk's dO, reverse mode gives
//   dUb = P^T dO + diag(Gc) K G',   dU = diag(beta) dUb,   dR = T^T dU,   dV = dR,
//   dA  = -tril_{-1}(dR U^T),   E1 = Gamma o tril(dO Ub^T),   E2 = Gamma o dA diag(beta),
//   dQ  = diag(gamma) dO S^T + E1 K,
//   dK  = E2 K - diag(gamma) dR S^T          (k_t as the row of A and R)
//       + E1^T Q + E2^T K + diag(Gc) Ub G'^T (k_i as a column of A and P, and in S'),
//   dbeta_t = U_t . dUb_t + sum_{t'} dA[t'][t] Gamma[t'][t] (k_t' . k_t),
//   dS  = gamma_C G' + Q^T diag(gamma) dO - K^T diag(gamma) dR.
// The state gradient is affine in G' with coefficients free of S, so it has
// segment maps like the forward's.  Gates: every gamma dependence goes
// through gamma_t q_t, gamma_t k_t, k_t / gamma_t and gamma_C, so with the
// two parts of dK above written dKp (rows) and dKm (columns),
//   dL/dl_t = q_t . dq_t + k_t . (dKp_t - dKm_t) + [t = C-1] <G', S'>,
// l_t = log gamma_t, and dlog alpha_s = sum_{t >= s} dL/dl_t within the
// chunk; <G', S'> = gamma_C <G', S> + sum_t Gc_t k_t . (G' Ub_t).  All
// quantities are bounded (only ratios gamma_t / gamma_i with i <= t occur).
//
// Launches (uniform batches; G segments of L tokens per sequence):
//   1-3  the forward sweep: segment maps, composition, then every chunk's
//        entering state S_c as bf16 tiles (delta_prefill.hip)
//   4    reverse chunk chain over segments 1..G-1 with the state gradient
//        started at 0: the constant parts c_g of the segments' reverse maps
//   5    reverse composition: G_end(g-1) = M_g^T G_end(g) + c_g from dS_T.
//        The G'-dependent part of dS above is A_c^T G' with A_c = gamma_C I -
//        K^T diag(beta Gc) T diag(gamma) K, the forward's state transition:
//        a segment's reverse map is the transpose of its forward map M_g,
//        which the forward sweep computes for every segment
//   6    reverse chunk chain from G_end(g): every chunk's G' as bf16 tiles,
//        and dS_0 from segment 0
//   7    every chunk independently: dq, dk, dv, dbeta, dalpha from (S_c, G'_c)
#include "common.hpp"
#include "delta_chunk.hpp"
#include "kernels.hpp"

namespace la {

namespace {

using dchunk::CH;
using dchunk::LT;
using dchunk::NT;
using dchunk::NWV;

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// ------------------------------------------------------------- reverse chain

template <int DK, int DV, bool MAP, bool GATED>
struct RC {
    // LDS layouts by use (gfx950 LDS probes): K is staged twice, group-
    // permuted for its row fragments (K G and P's builder) and natural for
    // the transpose loads of K^T dR; dO, P and T are read only with
    // transpose loads (natural, padded by 16, where those are
    // conflict-free); Q is read both ways and keeps the 8-element padding.
    using KF = RowLayout<DK + 16, true>;
    using KT = RowLayout<DK + 16>;
    using QL = RowLayout<DK + 8>;
    using OL = RowLayout<DV + 16>;
    using PL = RowLayout<CH + 16>;  // P and T
    static constexpr int KFS = CH * KF::LD * 2, KTS = CH * KT::LD * 2, QS = CH * QL::LD * 2, OS = CH * OL::LD * 2;
    static constexpr int TS = CH * PL::LD * 2, PS = CH * PL::LD * 2;
    static constexpr int BS = CH * 4 * (GATED ? 4 : 1);
    static constexpr int TOTAL = KFS + KTS + QS + OS + TS + PS + BS;
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
    static constexpr int XR = DK / 16;
    // Column tiles of the state gradient (c_g, or the gradient itself)
    static constexpr int NCN = DV / 16;
    static constexpr int NCT = NCN;
    static constexpr int SLOTS = (NCT + NWV - 1) / NWV;
};

// One workgroup runs one segment's chunks from last to first.  Each wave
// owns whole columns of the state gradient G (fp32, registers) and per chunk
//   dU[:, c] = beta o (P^T dO[:, c] + Gc o K G[:, c])
//   dR[:, c] = T^T dU[:, c]
//   G[:, c]  = gamma_C G[:, c] + (diag(gamma) Q)^T dO[:, c] - K^T diag(gamma) dR[:, c]
// with P, T (from the chunk records of the forward sweep) and the staged rows
// shared through LDS.
template <int DK, int DV, bool MAP, bool GATED>
__global__ __launch_bounds__(NT) void dlb_chain_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ beta,
    const float* __restrict__ alpha, const bf16_t* __restrict__ dO, const float* __restrict__ g_end,
    float* __restrict__ map_c, bf16_t* __restrict__ gst, float* __restrict__ dS0,
    const bf16_t* __restrict__ trec, SegMap sm) {
    using Y = RC<DK, DV, MAP, GATED>;
    using M = Mma<bf16_t>;
    using KF = typename Y::KF;
    using KT = typename Y::KT;
    using QL = typename Y::QL;
    using OL = typename Y::OL;
    using PL = typename Y::PL;
    constexpr int XR = Y::XR, SLOTS = Y::SLOTS;
    __shared__ __align__(16) unsigned char smem[Y::TOTAL];
    unsigned char* sp = smem;
    __bf16* Kf = reinterpret_cast<__bf16*>(sp);  sp += Y::KFS;
    __bf16* Kt = reinterpret_cast<__bf16*>(sp);  sp += Y::KTS;
    __bf16* Qs = reinterpret_cast<__bf16*>(sp);  sp += Y::QS;
    __bf16* Os = reinterpret_cast<__bf16*>(sp);  sp += Y::OS;
    __bf16* Ts = reinterpret_cast<__bf16*>(sp);  sp += Y::TS;
    __bf16* Ps = reinterpret_cast<__bf16*>(sp);  sp += Y::PS;
    float* Bs = reinterpret_cast<float*>(sp);
    float* Gl = Bs + CH;
    float* Ge = Gl + CH;
    float* Gc = Ge + CH;

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, li = lane & 15;
    const int w = wave_id(tid);
    __builtin_assume(w >= 0 && w < NT / 64);  // lets per-wave tile guards fold away
    const int G1 = MAP ? sm.G - 1 : sm.G;
    const int vh = blockIdx.x / G1;  // sequence * H + head
    const int seg = blockIdx.x % G1 + (MAP ? 1 : 0);
    const int nseq = vh / sm.H, h = vh % sm.H;
    const long slot = sm.slot<false>(nseq, h) + seg;
    const long row0 = h * sm.hs + sm.start<false>(nseq);
    const int NC = (sm.T + CH - 1) / CH;

    v4f X[SLOTS][XR];
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
        const int id = w + NWV * j;
        const int col = 16 * id + li;
#pragma unroll
        for (int i = 0; i < XR; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * i + 4 * g + r;
                X[j][i][r] = (!MAP && id < Y::NCT) ? g_end[(slot * DK + row) * DV + col] : 0.f;
            }
    }

    const int t0 = seg * sm.L;
    const int t_end = min((seg + 1) * sm.L, sm.T);
    const rsrc_t rk = make_rsrc(k + row0 * DK, (uint32_t)t_end * DK * 2);
    const rsrc_t rq = make_rsrc(q + row0 * DK, (uint32_t)t_end * DK * 2);
    const rsrc_t ro = make_rsrc(dO + row0 * DV, (uint32_t)t_end * DV * 2);
    const rsrc_t rb = make_rsrc(beta + row0, (uint32_t)t_end * 2);
    const rsrc_t ra = make_rsrc(GATED ? alpha + row0 : nullptr, GATED ? (uint32_t)t_end * 4 : 0u);
    ChunkRegs<bf16_t, DK, NT> kr, qr;
    ChunkRegs<bf16_t, DV, NT> orr;
    unsigned short bnext = 0;
    unsigned anext = 0;
    uint4 tnext;
    auto load_chunk = [&](int c) {
        kr.load_buf(rk, c, tid);
        qr.load_buf(rq, c, tid);
        orr.load_buf(ro, c, tid);
        tnext = dchunk::load_rec(trec + sm.chunk_rec<false>(nseq, h, c / CH, CH) * dchunk::kRecElems, tid);
        if (tid < CH) {
            bnext = __builtin_amdgcn_raw_buffer_load_b16(rb, (uint32_t)(c + tid) * 2, 0, 0);
            if constexpr (GATED) anext = __builtin_amdgcn_raw_buffer_load_b32(ra, (uint32_t)(c + tid) * 4, 0, 0);
        }
    };
    const int c_last = t0 + ((t_end - 1 - t0) / CH) * CH;
    load_chunk(c_last);
    dchunk::clear_upper<PL>(Ps, tid);  // upper blocks of P and of T (the records hold its lower tiles)
    dchunk::clear_upper<PL>(Ts, tid);
    for (int c0 = c_last; c0 >= t0; c0 -= CH) {
        // Lane indices from an opaque copy, re-derived every chunk: the many
        // per-lane LDS addresses built from them then live next to their uses
        // instead of being hoisted out of the loop (and spilled).
        int tid_v = threadIdx.x;
        asm volatile("" : "+v"(tid_v));
        const int tid = tid_v, lane = tid & 63, g = lane >> 4, li = lane & 15;
        const int n = min(CH, t_end - c0);
        if constexpr (!MAP) {  // the gradient of the state leaving this chunk
            const long ci = (long)vh * NC + c0 / CH;
#pragma unroll
            for (int j = 0; j < SLOTS; ++j) {
                const int id = w + NWV * j;
                if (id >= Y::NCN) continue;
#pragma unroll
                for (int i = 0; i < XR; ++i) dchunk::put_tile(gst + dchunk::tile_offset<DK, DV>(ci, id, i, lane), X[j][i]);
            }
        }
        stage_rows_raw<bf16_t, DK, NT, false, true>(kr, tid, Kf, KF::LD);
        stage_rows_raw<bf16_t, DK, NT>(kr, tid, Kt, KT::LD);
        stage_rows_raw<bf16_t, DK, NT>(qr, tid, Qs, QL::LD);
        stage_rows_raw<bf16_t, DV, NT>(orr, tid, Os, OL::LD);
        dchunk::stage_rec<PL>(Ts, tnext, tid);
        if (tid < CH) {
            Bs[tid] = bf16_to_f32(bnext);
            if constexpr (GATED) dchunk::gate_prefix(__uint_as_float(anext), tid, n, Gl, Ge, Gc);
        }
        if (c0 - CH >= t0) load_chunk(c0 - CH);
        __syncthreads();
        dchunk::build_P<DK, GATED, false, KF, QL, PL>(Kf, Qs, Gl, Ps, w, g, li);
        __syncthreads();
        if constexpr (GATED) {  // diag(gamma) Q for the dO term of the state gradient
            for (int e = tid; e < CH * DK / 8; e += NT) {
                const int row = e / (DK / 8), col = (e % (DK / 8)) * 8;
                v8bf x = *reinterpret_cast<const v8bf*>(&Qs[row * QL::LD + col]);
                const float s = Ge[row];
#pragma unroll
                for (int u = 0; u < 8; ++u) x[u] = M::cvt((float)x[u] * s);
                *reinterpret_cast<v8bf*>(&Qs[row * QL::LD + col]) = x;
            }
            __syncthreads();
        }

#pragma unroll
        for (int j = 0; j < SLOTS; ++j) {
            const int id = w + NWV * j;
            if (id >= Y::NCT) continue;
            v4f dU[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                v4f acc = zero4(), kg = zero4();
#pragma unroll
                for (int kb = 0; kb < CH / 32; ++kb) {
                    if (32 * kb + 31 < 16 * tt) continue;  // P^T is upper triangular
                    M::mma(acc, PL::tr(Ps, 32 * kb, 16 * tt, lane), OL::tr(Os, 32 * kb, 16 * id, lane));
                }
#pragma unroll
                for (int kb = 0; kb < DK / 32; ++kb)
                    M::mma(kg, KF::frag(Kf, 16 * tt + li, 32 * kb, g), M::from_tiles(X[j][2 * kb], X[j][2 * kb + 1]));
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = 16 * tt + 4 * g + r;
                    dU[tt][r] = Bs[s] * (acc[r] + (GATED ? Gc[s] : 1.f) * kg[r]);
                }
            }
            v4f dR[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                dR[tt] = zero4();
#pragma unroll
                for (int kb = 0; kb < CH / 32; ++kb) {
                    if (32 * kb + 31 < 16 * tt) continue;  // T^T is upper triangular
                    M::mma(dR[tt], PL::tr(Ts, 32 * kb, 16 * tt, lane), M::from_tiles(dU[2 * kb], dU[2 * kb + 1]));
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) dR[tt][r] *= GATED ? -Ge[16 * tt + 4 * g + r] : -1.f;
            }
            if constexpr (GATED) {
                const float gend = Ge[CH - 1];
#pragma unroll
                for (int i = 0; i < XR; ++i) X[j][i] *= gend;
            }
#pragma unroll
            for (int i = 0; i < XR; ++i) {
#pragma unroll
                for (int kb = 0; kb < CH / 32; ++kb)
                    M::mma(X[j][i], QL::tr(Qs, 32 * kb, 16 * i, lane), OL::tr(Os, 32 * kb, 16 * id, lane));
#pragma unroll
                for (int kb = 0; kb < CH / 32; ++kb)
                    M::mma(X[j][i], KT::tr(Kt, 32 * kb, 16 * i, lane), M::from_tiles(dR[2 * kb], dR[2 * kb + 1]));
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
        const int id = w + NWV * j;
        if (id >= Y::NCT) continue;
        float* dst;
        if constexpr (MAP) {
            dst = map_c + slot * DK * DV;
        } else {
            if (seg != 0 || !dS0) continue;
            dst = dS0 + (long)vh * DK * DV;
        }
        const int col = 16 * id + li;
#pragma unroll
        for (int i = 0; i < XR; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(16 * i + 4 * g + r) * DV + col] = X[j][i][r];
    }
}

// ------------------------------------------------------------- gradients

template <int DK, int DV, bool GATED>
struct GR {
    // Every bf16 matrix here is read as row fragments, most also with
    // transpose loads or as single elements: all group-permuted with 16
    // elements of padding (pcol), where fragment reads are single
    // conflict-free 16-byte reads and transpose reads cost what they do on
    // natural rows padded by 8 (gfx950 LDS probes).
    using KL = RowLayout<DK + 16, true>;  // K, Q
    using VL = RowLayout<DV + 16, true>;  // dO, V then U, dR, G' or S (DK rows)
    using PL = RowLayout<CH + 16, true>;  // T then E2, P then E1
    static constexpr int KS = CH * KL::LD * 2, QS = CH * KL::LD * 2, OS = CH * VL::LD * 2, US = CH * VL::LD * 2;
    static constexpr int RS = CH * VL::LD * 2;   // dR rows
    static constexpr int BG = DK * VL::LD * 2;   // G' or S rows
    static constexpr int TS = CH * PL::LD * 2, PS = CH * PL::LD * 2;
    // beta; per-wave partials of dbeta (rows, then E2 tiles) and of dL/dl;
    // per-wave partial sums; gates
    static constexpr int SM = (CH + NWV * CH + 10 * 16 + NWV * CH + 2 * NWV + (GATED ? 3 * CH : 0)) * 4;
    static constexpr int TOTAL = KS + QS + OS + US + RS + BG + TS + PS + SM;
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
    static constexpr int XR = DK / 16;
    static constexpr int NCN = DV / 16;
    static constexpr int TPW = DK / 32;  // (dk tile, token tile) pairs per wave in the row phase
};

// One workgroup per chunk.  Phases:
//   column phase (wave w < DV/16 owns value columns 16w..16w+15, with its
//     tiles of S_c and G'_c in registers): U, dUb, dU, dR as above; U and
//     dR rows to LDS, the U . dUb part of dbeta
//   E phase: E1 and E2 (the lower 16x16 tiles, bf16, over P and T in LDS)
//     and the column part of dbeta
//   row phase: dK's column part with G' rows in LDS, then S rows replace
//     them for dQ and dK's row part; dq, dk stored as transposed tiles (four
//     consecutive features per lane) and the gate sums dL/dl_t formed
template <int DK, int DV, bool GATED>
__global__ __launch_bounds__(NT) void dlb_grad_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ beta, const float* __restrict__ alpha, const bf16_t* __restrict__ dO,
    const bf16_t* __restrict__ sst, const bf16_t* __restrict__ gst, bf16_t* __restrict__ dq,
    bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, float* __restrict__ dbeta, float* __restrict__ dalpha,
    const bf16_t* __restrict__ trec, int HT, int T) {
    using Y = GR<DK, DV, GATED>;
    using M = Mma<bf16_t>;
    using KL = typename Y::KL;
    using VL = typename Y::VL;
    using PL = typename Y::PL;
    constexpr int XR = Y::XR, TPW = Y::TPW;
    __shared__ __align__(16) unsigned char smem[Y::TOTAL];
    unsigned char* sp = smem;
    __bf16* Ks = reinterpret_cast<__bf16*>(sp);  sp += Y::KS;
    __bf16* Qs = reinterpret_cast<__bf16*>(sp);  sp += Y::QS;
    __bf16* Os = reinterpret_cast<__bf16*>(sp);  sp += Y::OS;
    __bf16* Us = reinterpret_cast<__bf16*>(sp);  sp += Y::US;  // V, then U
    __bf16* Rs = reinterpret_cast<__bf16*>(sp);  sp += Y::RS;  // dR
    __bf16* Bg = reinterpret_cast<__bf16*>(sp);  sp += Y::BG;  // G' rows, then S rows
    __bf16* Ts = reinterpret_cast<__bf16*>(sp);  sp += Y::TS;  // T, then E2
    __bf16* Ps = reinterpret_cast<__bf16*>(sp);  sp += Y::PS;  // P, then E1
    // Partial sums live in per-wave (or per-tile) slots and are added in a
    // fixed order at the end, so results do not depend on wave timing.
    float* Bs = reinterpret_cast<float*>(sp);
    float* pB = Bs + CH;           // [wave][t]: U_t . dUb_t over the wave's columns
    float* pE = pB + NWV * CH;     // [E2 tile][column]: column sums of dA o Gamma o K K^T
    float* pL = pE + 10 * 16;      // [wave][t]: the wave's features of dL/dl_t
    float* pS = pL + NWV * CH;     // [wave]: <G', S> over the wave's columns
    float* pZ = pS + NWV;          // [wave]: sum Gc_t k_t . (G' Ub_t) over the wave's tiles
    float* Gl = pZ + NWV;
    float* Ge = Gl + CH;
    float* Gc = Ge + CH;

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, li = lane & 15;
    const int w = wave_id(tid);
    __builtin_assume(w >= 0 && w < NT / 64);  // lets per-wave tile guards fold away
    const int NC = (T + CH - 1) / CH;
    const long total = (long)HT * NC;

    // Persistent: workgroup b takes chunks b, b + gridDim.x, ...  The next
    // chunk's rows and per-token inputs are loaded into registers while this
    // one is computed; its state tiles once this chunk's are consumed.
    ChunkRegs<bf16_t, DK, NT> kr, qr;
    ChunkRegs<bf16_t, DV, NT> vr, orr;
    uint2 st[XR], gt[XR];  // this wave's tiles of S_c and G'_c
    unsigned short bnext = 0;
    unsigned anext = 0;
    uint4 tnext;  // this thread's 16 bytes of the chunk's T record (record index = chunk index)
    auto load_rows = [&](long c) {  // rows past the sequence end read as zero
        const int c0_ = (int)(c % NC) * CH, n_ = min(CH, T - c0_);
        const long r0 = (c / NC) * T + c0_;
        tnext = dchunk::load_rec(trec + c * dchunk::kRecElems, tid);
        // the last reads of these rows: non-temporal
        kr.template load_buf<kLastUse>(make_rsrc(k + r0 * DK, (uint32_t)n_ * DK * 2), 0, tid);
        qr.template load_buf<kLastUse>(make_rsrc(q + r0 * DK, (uint32_t)n_ * DK * 2), 0, tid);
        vr.template load_buf<kLastUse>(make_rsrc(v + r0 * DV, (uint32_t)n_ * DV * 2), 0, tid);
        orr.template load_buf<kLastUse>(make_rsrc(dO + r0 * DV, (uint32_t)n_ * DV * 2), 0, tid);
        if (tid < CH) {
            bnext = __builtin_amdgcn_raw_buffer_load_b16(make_rsrc(beta + r0, (uint32_t)n_ * 2), (uint32_t)tid * 2, 0, 0);
            if constexpr (GATED)
                anext = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(alpha + r0, (uint32_t)n_ * 4), (uint32_t)tid * 4,
                                                             0, 0);
        }
    };
    auto load_tiles = [&](long c) {
        if (w < Y::NCN) {
#pragma unroll
            for (int i = 0; i < XR; ++i) {
                st[i] = dchunk::get_tile(sst + dchunk::tile_offset<DK, DV>(c, w, i, lane));
                gt[i] = dchunk::get_tile(gst + dchunk::tile_offset<DK, DV>(c, w, i, lane));
            }
        }
    };
    long ci = blockIdx.x;
    if (ci < total) {
        load_rows(ci);
        load_tiles(ci);
    }
    // upper blocks of P and T (the records hold T's lower tiles; E1 reuses
    // P's lower tiles only, E2 writes T's zeros back with its own)
    dchunk::clear_upper<PL>(Ps, tid);
    dchunk::clear_upper<PL>(Ts, tid);
    for (; ci < total; ci += gridDim.x) {
    // lane indices re-derived per chunk from an opaque copy, so the per-lane
    // LDS addresses are not hoisted out of the loop and held (spilled)
    int tid_v = threadIdx.x;
    asm volatile("" : "+v"(tid_v));
    const int tid = tid_v, lane = tid & 63, g = lane >> 4, li = lane & 15;
    const int vh = (int)(ci / NC);
    const int c0 = (int)(ci % NC) * CH;
    const int n = min(CH, T - c0);
    const long row0 = (long)vh * T + c0;
    const long cn = ci + gridDim.x;  // the next chunk of this workgroup

    stage_rows_raw<bf16_t, DK, NT, false, true>(kr, tid, Ks, KL::LD);
    stage_rows_raw<bf16_t, DK, NT, false, true>(qr, tid, Qs, KL::LD);
    stage_rows_raw<bf16_t, DV, NT, false, true>(vr, tid, Us, VL::LD);
    stage_rows_raw<bf16_t, DV, NT, false, true>(orr, tid, Os, VL::LD);
    dchunk::stage_rec<PL>(Ts, tnext, tid);
    for (int e = tid; e < NWV * CH; e += NT) pL[e] = 0.f;  // waves write only their tokens
    if (tid < CH) {
        Bs[tid] = bf16_to_f32(bnext);
        if constexpr (GATED) dchunk::gate_prefix(__uint_as_float(anext), tid, n, Gl, Ge, Gc);
    }
    if (cn < total) load_rows(cn);
    __syncthreads();
    v4f kk[2];  // raw K K^T of the lower tiles w and w + 8, for dbeta
    dchunk::build_P<DK, GATED, true, KL, KL, PL>(Ks, Qs, Gl, Ps, w, g, li, kk);
    __syncthreads();

    // ---- column phase
    if (w < Y::NCN) {
        const int col = 16 * w + li;
        v4f U[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {  // R = V - diag(gamma) K S
            v4f ks = zero4();
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb)
                M::mma(ks, KL::frag(Ks, 16 * tt + li, 32 * kb, g), dchunk::tile_frag(st[2 * kb], st[2 * kb + 1]));
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = 16 * tt + 4 * g + r;
                U[tt][r] = (float)Us[VL::at(s, col)] - (GATED ? Ge[s] : 1.f) * ks[r];
            }
        }
        v4f Uo[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {  // U = T R
            Uo[tt] = zero4();
#pragma unroll
            for (int kb = 0; kb < CH / 32; ++kb) {
                if (32 * kb > 16 * tt + 15) continue;  // T is lower triangular
                M::mma(Uo[tt], PL::frag(Ts, 16 * tt + li, 32 * kb, g), M::from_tiles(U[2 * kb], U[2 * kb + 1]));
            }
        }
        v4f dUb[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {  // dUb = P^T dO + diag(Gc) K G'
            v4f acc = zero4(), kg = zero4();
#pragma unroll
            for (int kb = 0; kb < CH / 32; ++kb) {
                if (32 * kb + 31 < 16 * tt) continue;
                M::mma(acc, PL::tr(Ps, 32 * kb, 16 * tt, lane), VL::tr(Os, 32 * kb, 16 * w, lane));
            }
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb)
                M::mma(kg, KL::frag(Ks, 16 * tt + li, 32 * kb, g), dchunk::tile_frag(gt[2 * kb], gt[2 * kb + 1]));
#pragma unroll
            for (int r = 0; r < 4; ++r) dUb[tt][r] = acc[r] + (GATED ? Gc[16 * tt + 4 * g + r] : 1.f) * kg[r];
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)  // dbeta_t += U_t . dUb_t over this wave's columns
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = row16_sum(Uo[tt][r] * dUb[tt][r]);
                if (li == 0) pB[w * CH + 16 * tt + 4 * g + r] = x;
                dUb[tt][r] *= Bs[16 * tt + 4 * g + r];  // dU
            }
        v4f dR[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {  // dR = T^T dU
            dR[tt] = zero4();
#pragma unroll
            for (int kb = 0; kb < CH / 32; ++kb) {
                if (32 * kb + 31 < 16 * tt) continue;
                M::mma(dR[tt], PL::tr(Ts, 32 * kb, 16 * tt, lane), M::from_tiles(dUb[2 * kb], dUb[2 * kb + 1]));
            }
        }
        if constexpr (GATED) {  // <G', S> over this wave's columns
            float x = 0.f;
#pragma unroll
            for (int i = 0; i < XR; ++i) {
                const v4f a = dchunk::tile_f32(st[i]), b = dchunk::tile_f32(gt[i]);
                x += a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
            }
            x = row16_sum(x);
            x += __shfl_xor(x, 16);
            x += __shfl_xor(x, 32);
            if (lane == 0) pS[w] = x;
        }
        // U and dR rows (own columns; this wave alone read them as V), G' rows
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = 16 * tt + 4 * g + r;
                Us[VL::at(s, col)] = M::cvt(Uo[tt][r]);
                Rs[VL::at(s, col)] = M::cvt(dR[tt][r]);
            }
#pragma unroll
        for (int i = 0; i < XR; ++i) {
            const bf16_t e[4] = {(bf16_t)(gt[i].x & 0xffffu), (bf16_t)(gt[i].x >> 16), (bf16_t)(gt[i].y & 0xffffu),
                                 (bf16_t)(gt[i].y >> 16)};
#pragma unroll
            for (int r = 0; r < 4; ++r) Bg[VL::at(16 * i + 4 * g + r, col)] = __builtin_bit_cast(__bf16, e[r]);
        }
    }
    __syncthreads();

    // ---- dv rows, then E1, E2 and the column part of dbeta
    for (int e = tid; e < CH * DV / 4; e += NT) {  // 8-byte pieces: whole 4-column groups of the permuted rows
        const int row = e / (DV / 4), c4 = (e % (DV / 4)) * 4;
        if (row < n) *reinterpret_cast<uint2*>(dv + (row0 + row) * DV + c4) = *reinterpret_cast<const uint2*>(&Rs[VL::at(row, c4)]);
    }
    // E2 tile j goes to wave j % 8 (which holds its K K^T from the inverse),
    // E1 tiles to the waves with fewer: at most three tiles per wave.
    auto e_tile = [&](int j, bool e2, const v4f& kkt) {
        int bt, bi;
        dchunk::lower_tile(j, bt, bi);
        v4f acc = zero4();
        const __bf16* lhs = e2 ? Rs : Os;
#pragma unroll
        for (int kb = 0; kb < DV / 32; ++kb)
            M::mma(acc, VL::frag(lhs, 16 * bt + li, 32 * kb, g), VL::frag(Us, 16 * bi + li, 32 * kb, g));
        const int i = 16 * bi + li;
        if (!e2) {  // E1 = Gamma o tril(dO U^T) diag(beta)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * bt + 4 * g + r;
                const float ratio = GATED ? __expf(Gl[t] - Gl[i]) : 1.f;
                Ps[PL::at(t, i)] = M::cvt(i <= t ? Bs[i] * ratio * acc[r] : 0.f);
            }
        } else {  // dA = -tril_{-1}(dR U^T); E2 = Gamma o dA diag(beta)
            float cs = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * bt + 4 * g + r;
                const float ratio = GATED ? __expf(Gl[t] - Gl[i]) : 1.f;
                const float ga = -acc[r] * ratio;
                Ts[PL::at(t, i)] = M::cvt(i < t ? Bs[i] * ga : 0.f);
                cs += i < t ? ga * kkt[r] : 0.f;
            }
            cs += __shfl_xor(cs, 16);
            cs += __shfl_xor(cs, 32);
            if (g == 0) pE[j * 16 + li] = cs;
        }
    };
    e_tile(w, true, kk[0]);
    if (w < 2) e_tile(w + NWV, true, kk[1]);
    if (w >= 2) e_tile(w - 2, false, kk[0]);
    if (w >= 2 && w < 6) e_tile(w + 4, false, kk[0]);
    __syncthreads();

    // ---- row phase.  Wave w: dk tile it, token tiles tb .. tb + TPW - 1;
    // accumulators hold transposed tiles (rows = features, column = token).
    const int it = w % (DK / 16), tb = (w / (DK / 16)) * TPW;
    v4f km[TPW];
    float zs = 0.f;
    // operands of the wave's feature tile, shared by its token tiles
    M::frag qT[CH / 32], kT[CH / 32], rf[DV / 32];
#pragma unroll
    for (int kb = 0; kb < CH / 32; ++kb) {
        qT[kb] = KL::tr(Qs, 32 * kb, 16 * it, lane);
        kT[kb] = KL::tr(Ks, 32 * kb, 16 * it, lane);
    }
#pragma unroll
    for (int kb = 0; kb < DV / 32; ++kb) rf[kb] = VL::frag(Bg, 16 * it + li, 32 * kb, g);  // G' rows
#pragma unroll
    for (int u = 0; u < TPW; ++u) {  // dKm = E1^T Q + E2^T K + diag(Gc beta) U G'^T
        const int tt = tb + u;
        km[u] = zero4();
#pragma unroll
        for (int kb = 0; kb < CH / 32; ++kb) {
            if (32 * kb + 31 < 16 * tt) continue;  // E1, E2 vanish above the diagonal
            M::mma(km[u], qT[kb], PL::tr(Ps, 32 * kb, 16 * tt, lane));
            M::mma(km[u], kT[kb], PL::tr(Ts, 32 * kb, 16 * tt, lane));
        }
        v4f g3 = zero4();
#pragma unroll
        for (int kb = 0; kb < DV / 32; ++kb) M::mma(g3, rf[kb], VL::frag(Us, 16 * tt + li, 32 * kb, g));
        const int t = 16 * tt + li;
        const float sc = Bs[t] * (GATED ? Gc[t] : 1.f);
        const v4bf kv = *reinterpret_cast<const v4bf*>(&Ks[KL::at(t, 16 * it + 4 * g)]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            km[u][r] += sc * g3[r];
            zs += (float)kv[r] * sc * g3[r];
        }
    }
    if constexpr (GATED) {
        zs = row16_sum(zs);
        zs += __shfl_xor(zs, 16);
        zs += __shfl_xor(zs, 32);
        if (lane == 0) pZ[w] = zs;
    }
    __syncthreads();
    if (w < Y::NCN) {  // S rows replace G' rows
#pragma unroll
        for (int i = 0; i < XR; ++i) {
            const bf16_t e[4] = {(bf16_t)(st[i].x & 0xffffu), (bf16_t)(st[i].x >> 16), (bf16_t)(st[i].y & 0xffffu),
                                 (bf16_t)(st[i].y >> 16)};
#pragma unroll
            for (int r = 0; r < 4; ++r) Bg[VL::at(16 * i + 4 * g + r, 16 * w + li)] = __builtin_bit_cast(__bf16, e[r]);
        }
    }
    if (cn < total) load_tiles(cn);  // this chunk's tiles are consumed
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < DV / 32; ++kb) rf[kb] = VL::frag(Bg, 16 * it + li, 32 * kb, g);  // S rows
    float xl[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {  // dQ = diag(gamma) dO S^T + E1 K;  dKp = E2 K - diag(gamma) dR S^T
        const int tt = tb + u;
        v4f a1 = zero4(), a2 = zero4();
#pragma unroll
        for (int kb = 0; kb < DV / 32; ++kb) {
            M::mma(a1, rf[kb], VL::frag(Os, 16 * tt + li, 32 * kb, g));
            M::mma(a2, rf[kb], VL::frag(Rs, 16 * tt + li, 32 * kb, g));
        }
        const int t = 16 * tt + li;
        const float ge = GATED ? Ge[t] : 1.f;
        v4f dqv = a1 * ge, kp = a2 * (-ge);
#pragma unroll
        for (int kb = 0; kb < CH / 32; ++kb) {
            if (32 * kb > 16 * tt + 15) continue;  // E1, E2 rows end at the diagonal
            M::mma(dqv, kT[kb], PL::frag(Ps, 16 * tt + li, 32 * kb, g));
            M::mma(kp, kT[kb], PL::frag(Ts, 16 * tt + li, 32 * kb, g));
        }
        if (t < n) {
            uint2 pq, pk;
            pq.x = pack_bf16x2(dqv[0], dqv[1]);
            pq.y = pack_bf16x2(dqv[2], dqv[3]);
            pk.x = pack_bf16x2(kp[0] + km[u][0], kp[1] + km[u][1]);
            pk.y = pack_bf16x2(kp[2] + km[u][2], kp[3] + km[u][3]);
            *reinterpret_cast<uint2*>(dq + (row0 + t) * DK + 16 * it + 4 * g) = pq;
            *reinterpret_cast<uint2*>(dk + (row0 + t) * DK + 16 * it + 4 * g) = pk;
        }
        if constexpr (GATED) {  // q_t . dq_t + k_t . (dKp_t - dKm_t), this wave's features
            const v4bf qv = *reinterpret_cast<const v4bf*>(&Qs[KL::at(t, 16 * it + 4 * g)]);
            const v4bf kv = *reinterpret_cast<const v4bf*>(&Ks[KL::at(t, 16 * it + 4 * g)]);
            float x = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) x += (float)qv[r] * dqv[r] + (float)kv[r] * (kp[r] - km[u][r]);
            xl[u] = x;
        }
    }
    if constexpr (GATED) {  // the four lane groups hold different features of token 16 tt + li
#pragma unroll
        for (int u = 0; u < TPW; ++u) xl[u] += __shfl_xor(xl[u], 16);
#pragma unroll
        for (int u = 0; u < TPW; ++u) xl[u] += __shfl_xor(xl[u], 32);
        if (g == 0) {
#pragma unroll
            for (int u = 0; u < TPW; ++u) pL[w * CH + 16 * (tb + u) + li] = xl[u];
        }
    }
    __syncthreads();

    if (tid < CH) {
        const int t = tid;
        float db = 0.f;
        for (int u = 0; u < Y::NCN; ++u) db += pB[u * CH + t];
        for (int j = 0; j < 10; ++j) {  // E2 tiles whose columns hold t
            int bt, bi;
            dchunk::lower_tile(j, bt, bi);
            if (bi == t / 16) db += pE[j * 16 + t % 16];
        }
        if (t < n) dbeta[row0 + t] = db;
        if constexpr (GATED) {
            float x = 0.f, s0 = 0.f, z = 0.f;
            for (int u = 0; u < NWV; ++u) {
                x += pL[u * CH + t];
                z += pZ[u];
            }
            for (int u = 0; u < Y::NCN; ++u) s0 += pS[u];
            x += t == CH - 1 ? Ge[CH - 1] * s0 + z : 0.f;
#pragma unroll
            for (int off = 1; off < CH; off <<= 1) {  // suffix sums: dlog alpha_t = sum_{t' >= t} dL/dl_t'
                const float y = __shfl_down(x, off);
                x += t + off < CH ? y : 0.f;
            }
            if (t < n) {
                const float a = alpha[row0 + t];
                // the forward clamps log alpha at -20: no gradient below it
                dalpha[row0 + t] = logf(a) > -20.f ? x / a : 0.f;
            }
        }
    }
    __syncthreads();  // the partial sums and gates are read above before the next chunk overwrites them
    }
}

template <int DK, int DV, bool GATED>
hipError_t launch_typed(const bf16_t* q, const bf16_t* k, const bf16_t* v, const bf16_t* beta, const float* alpha,
                        const float* S0, const bf16_t* dO, const float* dS_T, bf16_t* dq, bf16_t* dk, bf16_t* dv,
                        float* dbeta, float* dalpha, float* dS0, const SegMap& sm, float* ws, hipStream_t stream,
                        bool after_forward) {
    const size_t slots = (size_t)sm.H * sm.NS;
    const int HT = sm.N * sm.H, NC = (sm.T + CH - 1) / CH;
    float* map_c = ws;                       // forward N_g, then c_g
    float* map_mt = map_c + slots * DK * DV; // forward M_g (the reverse composition reads it transposed)
    float* g_end = map_mt + slots * DK * DK; // forward segment states, then segment-end gradients
    // the chunk records of T left by the forward sweep, then the chunk-state tiles
    const bf16_t* trec = reinterpret_cast<const bf16_t*>(g_end + slots * DK * DV);
    bf16_t* sst = static_cast<bf16_t*>(delta_backward_states(ws, sm, DK, DV));
    bf16_t* gst = sst + (size_t)HT * NC * DK * DV;
    hipError_t err;
    if (!after_forward) {  // else a training forward left these arrays and the chunk states in ws
        err = launch_delta_states(q, k, v, beta, alpha, S0, sst, sm, DK, DV, ws, stream);
        if (err != hipSuccess) return err;
    }
    if (sm.G > 1) {
        dlb_chain_kernel<DK, DV, true, GATED><<<dim3(HT * (sm.G - 1)), dim3(NT), 0, stream>>>(
            q, k, beta, alpha, dO, nullptr, map_c, nullptr, nullptr, trec, sm);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if ((err = launch_delta_compose_rev(map_c, map_mt, dS_T, g_end, sm, DK, DV, stream)) != hipSuccess) return err;
    dlb_chain_kernel<DK, DV, false, GATED><<<dim3(HT * sm.G), dim3(NT), 0, stream>>>(q, k, beta, alpha, dO, g_end,
                                                                                 nullptr, gst, dS0, trec, sm);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    // one workgroup per compute unit (the LDS allows one), each looping over chunks
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 256;  // the grid size only sets the work split
    const long total = (long)HT * NC;
    const int grid = (int)(total < cus ? total : cus);
    dlb_grad_kernel<DK, DV, GATED><<<dim3(grid), dim3(NT), 0, stream>>>(q, k, v, beta, alpha, dO, sst, gst, dq, dk, dv,
                                                                       dbeta, dalpha, trec, HT, sm.T);
    return hipGetLastError();
}

}  // namespace

size_t delta_backward_ws_floats(long slots, long recs, int HT, int T, int dk, int dv) {
    const size_t nc = (size_t)(T + CH - 1) / CH;
    // the forward's arrays (per slot, per chunk record), then S_c and G'_c
    // tiles (bf16, two per float)
    return delta_ws_floats(slots, recs, dk, dv) + (size_t)HT * nc * dk * dv;
}

void* delta_backward_states(float* ws, const SegMap& sm, int dk, int dv) {
    const long slots = (long)sm.H * sm.NS;
    return ws + delta_ws_floats(slots, (long)sm.H * sm.chunk_recs_per_head(CH), dk, dv);
}

hipError_t launch_delta_backward(const void* q, const void* k, const void* v, const void* beta, const float* alpha,
                                 const float* S0, const void* dO, const float* dS_T, void* dq, void* dk_, void* dv_,
                                 float* dbeta, float* dalpha, float* dS0, const SegMap& sm, int dk, int dv, int dtype,
                                 float* ws, hipStream_t stream, bool after_forward) {
    if (dtype != 1 || sm.packed()) return hipErrorInvalidValue;
    const bf16_t* qb = static_cast<const bf16_t*>(q);
    const bf16_t* kb = static_cast<const bf16_t*>(k);
    const bf16_t* vb = static_cast<const bf16_t*>(v);
    const bf16_t* bb = static_cast<const bf16_t*>(beta);
    const bf16_t* ob = static_cast<const bf16_t*>(dO);
    bf16_t* dqb = static_cast<bf16_t*>(dq);
    bf16_t* dkb = static_cast<bf16_t*>(dk_);
    bf16_t* dvb = static_cast<bf16_t*>(dv_);
#define DLB_CASE(A, B)                                                                                         \
    if (dk == A && dv == B)                                                                                    \
        return alpha ? launch_typed<A, B, true>(qb, kb, vb, bb, alpha, S0, ob, dS_T, dqb, dkb, dvb, dbeta,     \
                                                dalpha, dS0, sm, ws, stream, after_forward)                    \
                     : launch_typed<A, B, false>(qb, kb, vb, bb, nullptr, S0, ob, dS_T, dqb, dkb, dvb, dbeta,  \
                                                 nullptr, dS0, sm, ws, stream, after_forward);
    DLB_CASE(64, 64)
    DLB_CASE(64, 128)
    DLB_CASE(128, 64)
    DLB_CASE(128, 128)
#undef DLB_CASE
    return hipErrorInvalidValue;
}

}  // namespace la
