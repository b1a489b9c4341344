// Delta-rule fast-weight memory, chunked prefill on gfx950.
//
// The rule ("AIGC 基本功｜线性、循环与记忆架构-LinearMem" §03 "从累加改成纠错";
// "手撕：递推与记忆模型" "Delta-rule fast weight"):
//   S_t = S_{t-1} + beta_t k_t (v_t^T - k_t^T S_{t-1}),   read o_t = S_t^T q_t.
//
// Chunked form.  Unrolling the rule over a chunk of C = 64 tokens with state
// S at the chunk start, the corrections u_t = v_t - S_{t-1}^T k_t satisfy the
// unit lower-triangular system
//   (I + A) U = V - K S,        A[t][i] = beta_i (k_t . k_i)  for i < t,
// so with T = (I + A)^{-1}, W = T K and U_v = T V:
//   U   = U_v - W S
//   O   = Q S + tril(Q K^T) (beta o U)          (write-then-read: diagonal kept)
//   S' += K^T (beta o U)
// (beta o U scales row t of U by beta_t).  T, W and U_v depend only on the
// chunk's own keys, values and betas; the state enters through W S alone.
// T is built once per chunk by a parallel pass (delta_tinv, the construction
// in delta_chunk.hpp: 16x16 diagonal blocks by forward substitution, then
// 2x2 block doubling in fp32) into per-chunk records, which the serial chunk
// loops below load with each chunk's rows.
//
// Sequence parallelism.  Over a segment of chunks the rule is affine in the
// incoming state: S_out = M_g S_in + N_g.  Running the same chunk recurrence
// on a state started at 0 with the segment's values gives N_g; running it on a
// state started at I with zero values gives M_g.  Each state column evolves
// independently, so both ride in one workgroup as extra columns and share the
// chunk's T and W.  Four launches:
//   delta_tinv        every chunk's T record
//   delta_chunk<MAP>  (M_g, N_g) for every segment but the last
//   delta_compose     S_in(g+1) = M_g S_in(g) + N_g, fp32 MFMA, serial in g
//   delta_chunk<OUT>  the chunk loop from S_in(g), writing O (and S_T last)
//
// Forgetting gate (LinearMem §03: decay the old state by alpha_t, then take
// the error against the decayed state; the Gated DeltaNet rule):
//   S_t = alpha_t S_{t-1} + beta_t k_t (v_t - alpha_t S_{t-1}^T k_t)^T.
// With chunk-local products gamma_t = alpha_{c0} ... alpha_t the chunk's
// state is S_t = gamma_t S + sum_{i<=t} (gamma_t/gamma_i) beta_i k_i u_i^T, so
// the same scheme holds with decay ratios folded in:
//   A[t][i] = (gamma_t/gamma_i) beta_i (k_t . k_i),     W = T diag(gamma) K,
//   O = diag(gamma) Q S + (tril(Q K^T) o Gamma)(beta o U),  Gamma[t][i] = gamma_t/gamma_i,
//   S' = gamma_C S + K^T diag(beta gamma_C / gamma) U.
// Ratios are exponentials of differences of chunk-local cumulative log-gates
// (each log clamped at -20), so no ratio divides by an underflowed product.
// The segment maps stay affine in the incoming state, so the launches are
// unchanged.
//
// Serving input transforms (LinearMem §05 and §08: the L2 normalisation of
// q and k and the beta transform run inside the kernel): with kNormQK each
// staged q and k row is scaled to unit L2 norm; with kBetaSigmoid beta holds
// logits and is passed through a sigmoid.  pred (optional) receives the
// prediction made before each write, v_t - u_t = (decayed S_{t-1})^T k_t
// ("手撕：递推与记忆模型", "Delta-rule fast weight", which reads first and
// then writes with the error).
#include "common.hpp"
#include "delta_chunk.hpp"
#include "kernels.hpp"
#include "la_chunked.hpp"

namespace la {

namespace {

constexpr int CH = kChunk;
constexpr int NT = 512;  // eight waves
constexpr int NWV = 8;

// What a run of delta_chunk computes: the segment maps, the outputs, or (for
// the backward pass) only the state entering every chunk.
enum { kMap = 0, kOut = 1, kStates = 2 };

template <int DK, int NS, int MODE, bool GATED, int NWV = 8>
struct DL {
    static constexpr bool OUT = MODE == kOut, MAP = MODE == kMap;
    // Row strides (bf16 elements), by how each matrix is read (LDS probes on
    // gfx950): matrices read as row fragments (W, Q, T, P) are stored
    // group-permuted (pcol) with 16 elements of padding, so a fragment is one
    // conflict-free 16-byte read; matrices read only with transpose loads (V,
    // K) keep the natural layout, also padded by 16, where those reads are
    // conflict-free.  The output and state passes read K both ways and stage
    // it twice: natural (Ks) and permuted (Kf, for the row fragments).
    static constexpr int LQ = DK + 16;  // K rows (natural and permuted)
    static constexpr int LW = DK + 16;  // W and Q rows (permuted)
    static constexpr int LV = NS + 16;  // V rows
    static constexpr int LT = CH + 16;  // T and P rows (permuted)
    static constexpr int KS = CH * LQ * 2;          // K_c rows, natural (transpose loads)
    static constexpr int KF = MAP ? 0 : CH * LQ * 2;  // K_c rows, permuted (row fragments)
    static constexpr int WS = MAP ? CH * LW * 2 : 0;  // W rows (map pass)
    static constexpr int QS = OUT ? CH * LW * 2 : 0;
    static constexpr int VS = CH * LV * 2;          // V_c rows (read transposed)
    static constexpr int TS = CH * LT * 2;          // T (bf16, from the chunk's record)
    static constexpr int PS = OUT ? CH * LT * 2 : 0;  // tril(Q K^T), rows = queries
    static constexpr int BS = CH * 4 * (GATED ? 4 : 1);  // beta; gated: log-gates, gamma, gamma_C/gamma (fp32)
    static constexpr int TOTAL = KS + KF + WS + QS + VS + TS + PS + BS;
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
    static constexpr int XR = DK / 16;              // dk row tiles of a state column
    // State column tiles: OUT and STATES carry S (NS columns); MAP carries N
    // (NS columns, zero start, with values) and M (DK columns, identity
    // start, no values).  Wave w owns tiles w, w + 8, ...
    static constexpr int NCN = NS / 16;
    static constexpr int NCT = MAP ? NCN + DK / 16 : NCN;
    static constexpr int SLOTS = (NCT + NWV - 1) / NWV;
    static constexpr int W_TPW = 4 * XR / NWV;      // W^T tiles per wave (map pass)
};

// Chunk rows of a [T][D] bf16 matrix into LDS scaled to unit L2 norm (a zero
// row stays zero).  The D/8 threads holding a row are consecutive lanes, so
// the row's sum of squares is a shuffle reduction within their group.
template <int D, int NTH = NT, bool SPLIT8 = false, bool PERM = false>
__device__ __forceinline__ void stage_rows_l2(const ChunkRegs<bf16_t, D, NTH>& cr, int tid, __bf16* rm, int ld) {
    constexpr int TPR = D / 8;
#pragma unroll
    for (int j = 0; j < ChunkRegs<bf16_t, D, NTH>::NV; ++j) {
        const int row = ChunkRegs<bf16_t, D, NTH>::row_of(j, tid);
        const int col = ChunkRegs<bf16_t, D, NTH>::col_of(j, tid);
        float x[8], ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            x[e] = cr.get(j, e);
            ss += x[e] * x[e];
        }
#pragma unroll
        for (int m = 1; m < TPR; m <<= 1) ss += __shfl_xor(ss, m);
        const float inv = ss > 0.f ? __builtin_amdgcn_rsqf(ss) : 0.f;
        uint4 y;
        y.x = pack_bf16x2(x[0] * inv, x[1] * inv);
        y.y = pack_bf16x2(x[2] * inv, x[3] * inv);
        y.z = pack_bf16x2(x[4] * inv, x[5] * inv);
        y.w = pack_bf16x2(x[6] * inv, x[7] * inv);
        if constexpr (PERM) {  // group-permuted rows (pcol)
            *reinterpret_cast<uint2*>(rm + row * ld + pcol(col)) = make_uint2(y.x, y.y);
            *reinterpret_cast<uint2*>(rm + row * ld + pcol(col + 4)) = make_uint2(y.z, y.w);
        } else if constexpr (SPLIT8) {
            uint2* d = reinterpret_cast<uint2*>(rm + row * ld + col);
            d[0] = make_uint2(y.x, y.y);
            d[1] = make_uint2(y.z, y.w);
        } else {
            *reinterpret_cast<uint4*>(rm + row * ld + col) = y;
        }
    }
}

using dchunk::lower_tile;

using dchunk::kRecElems;    // one chunk record: T's ten lower 16 x 16 tiles
using dchunk::kRecPieces;  // its 16-byte pieces

// T = (I + A)^{-1} of every chunk: the state-free, latency-bound part of
// the chunk recurrence (for the gated rule with the decay ratios in A), done once per
// chunk by a fully parallel pass (one workgroup per chunk record) instead of
// inside every serial chunk loop that needs it.  Rows past the sequence end
// are zero, as in the loops; the input transforms (kNormQK on k,
// kBetaSigmoid on beta) are applied as there.
template <int DK, bool GATED, bool PACKED>
__global__ __launch_bounds__(NT) void delta_tinv_kernel(const bf16_t* __restrict__ k, const bf16_t* __restrict__ beta,
                                                        const float* __restrict__ alpha, bf16_t* __restrict__ trec,
                                                        int flags, SegMap sm) {
    // K is read only as row fragments here (K K^T tiles): group-permuted
    // rows padded by 16 (pcol), one conflict-free 16-byte read a fragment
    // K is dead once A = K K^T is formed, so A takes K's LDS (one buffer of
    // the larger size): 35 KB instead of 52 KB per workgroup, four
    // workgroups per CU instead of three.
    using KL = RowLayout<DK + 16, true>;
    constexpr int LQ = KL::LD, LT = dchunk::LT, LF = dchunk::LF;
    constexpr int KA_BYTES = CH * LQ * 2 > CH * LF * 4 ? CH * LQ * 2 : CH * LF * 4;
    __shared__ __align__(16) unsigned char KAs[KA_BYTES];
    __bf16* Ks = reinterpret_cast<__bf16*>(KAs);
    float* Af = reinterpret_cast<float*>(KAs);
    __shared__ __align__(16) __bf16 Ts[CH * LT];
    __shared__ __align__(16) float Ad[4 * 256];
    __shared__ __align__(16) float Yf[4 * 256];
    __shared__ float Bs[CH], Gl[CH], Ge[CH], Gc[CH];
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, li = lane & 15;
    const int w = wave_id(tid);
    __builtin_assume(w >= 0 && w < NT / 64);  // lets per-wave tile guards fold away
    const long rec = blockIdx.x;
    int n, h, c;
    if constexpr (!PACKED) {
        const int ncs = (sm.T + CH - 1) / CH;
        const int vh = (int)(rec / ncs);
        c = (int)(rec % ncs);
        n = vh / sm.H;
        h = vh % sm.H;
    } else {  // invert the record map: the largest n with floor(start(n) / C) + n <= r
        const int R = sm.T / CH + sm.N;
        h = (int)(rec / R);
        const int r = (int)(rec % R);
        int lo = 0, hi = sm.N - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sm.start<true>(mid) / CH + mid <= r) lo = mid;
            else hi = mid - 1;
        }
        n = lo;
        c = r - (int)(sm.start<true>(n) / CH) - n;
        if (c < 0 || c * CH >= sm.length<true>(n)) return;  // a gap between sequences
    }
    const int c0 = c * CH;
    const int rows = min(CH, sm.length<PACKED>(n) - c0);
    const long row0 = h * sm.hs + sm.start<PACKED>(n) + c0;
    ChunkRegs<bf16_t, DK, NT> kr;
    kr.load_buf(make_rsrc(k + row0 * DK, (uint32_t)rows * DK * 2), 0, tid);
    if (flags & kNormQK) stage_rows_l2<DK, NT, false, true>(kr, tid, Ks, LQ);
    else stage_rows_raw<bf16_t, DK, NT, false, true>(kr, tid, Ks, LQ);
    if (tid < CH) {
        const float braw = bf16_to_f32(
            __builtin_amdgcn_raw_buffer_load_b16(make_rsrc(beta + row0, (uint32_t)rows * 2), (uint32_t)tid * 2, 0, 0));
        Bs[tid] = (flags & kBetaSigmoid) ? 1.f / (1.f + __expf(-braw)) : braw;
        if constexpr (GATED) {
            const unsigned a = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(alpha + row0, (uint32_t)rows * 4),
                                                                    (uint32_t)tid * 4, 0, 0);
            dchunk::gate_prefix(__uint_as_float(a), tid, rows, Gl, Ge, Gc);
        }
    }
    dchunk::clear_upper(Ts, tid);
    __syncthreads();
    dchunk::build_T<DK, GATED, false, false, KL, true>(Ks, nullptr, Bs, Gl, Af, Ad, Yf, Ts, nullptr, w, g, li);
    // the record: T's lower tiles, one 16-byte piece per thread
    if (tid < kRecPieces) {
        int row, col;
        dchunk::rec_piece(tid, row, col);
        *reinterpret_cast<uint4*>(trec + rec * kRecElems + tid * 8) =
            *reinterpret_cast<const uint4*>(&Ts[row * LT + col]);
    }
}

// One workgroup runs one segment's chunk loop.  The state-dependent part of
// a chunk is column-parallel (state columns evolve independently), so each
// wave owns whole state columns and keeps them, its corrections U and its
// outputs in registers:
//   U[:, c]  = U_v[:, c] - W S[:, c]            (W S from registers: S tiles are B operands)
//   O^T[c]   = S[:, c]^T Q^T + (beta o U[:, c])^T P^T   (OUT; S before the update)
//   S[:, c] += K^T (beta o U[:, c])
// The shared, state-free part (A, P, T, W) is computed by all waves through
// LDS.  MAP runs N and M in the same workgroup, so T and W are built once.
template <int DK, int NS, int MODE, bool GATED, bool PACKED, int NWV = 8>
__global__ __launch_bounds__(NWV * 64) void delta_chunk_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ beta, const float* __restrict__ alpha, bf16_t* __restrict__ o,
    const float* __restrict__ state_in, float* __restrict__ map_n, float* __restrict__ map_m,
    float* __restrict__ S_out, bf16_t* __restrict__ pred, bf16_t* __restrict__ states,
    const bf16_t* __restrict__ trec, int flags, SegMap sm) {
    constexpr bool OUT = MODE == kOut, MAP = MODE == kMap;
    static_assert(MODE != kStates || !PACKED, "chunk states are for uniform batches");
    constexpr int NT = NWV * 64;  // this instantiation's threads (eight or sixteen waves)
    using Y = DL<DK, NS, MODE, GATED, NWV>;
    using M = Mma<bf16_t>;
    typedef M::frag frag;
    constexpr int LQ = Y::LQ, LV = Y::LV, LT = Y::LT, XR = Y::XR, SLOTS = Y::SLOTS;
    __shared__ __align__(16) unsigned char smem[Y::TOTAL];
    unsigned char* sp = smem;
    __bf16* Ks = reinterpret_cast<__bf16*>(sp);  sp += Y::KS;
    __bf16* Kf = reinterpret_cast<__bf16*>(sp);  sp += Y::KF;
    __bf16* Ws = reinterpret_cast<__bf16*>(sp);  sp += Y::WS;
    __bf16* Qs = reinterpret_cast<__bf16*>(sp);  sp += Y::QS;
    __bf16* Vs = reinterpret_cast<__bf16*>(sp);  sp += Y::VS;
    __bf16* Ts = reinterpret_cast<__bf16*>(sp);  sp += Y::TS;
    __bf16* Ps = reinterpret_cast<__bf16*>(sp);  sp += Y::PS;
    float* Bs = reinterpret_cast<float*>(sp);
    float* Gl = Bs + CH;  // gated: chunk-local cumulative log-gate
    float* Ge = Gl + CH;  //        gamma_t = exp(Gl[t])
    float* Gc = Ge + CH;  //        gamma_C / gamma_t

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, li = lane & 15;
    const int w = wave_id(tid);
    __builtin_assume(w >= 0 && w < NWV);  // lets per-wave tile guards fold away
    // This workgroup's (head, sequence, segment).  The forward's MAP skips
    // the last segment of every sequence (its result is the sequence's final
    // state); the backward's forward sweep also wants that segment's M (the
    // reverse composition runs on M^T), so for uniform batches MAP covers the
    // segments the grid holds: G - 1 or G per sequence.
    int h, nseq, seg;
    if constexpr (!PACKED) {  // (sequence, head)-major, segments consecutive
        const int G1 = MAP ? (int)(gridDim.x / ((unsigned)sm.N * sm.H)) : sm.G;
        const int vh = blockIdx.x / G1;
        seg = blockIdx.x % G1;
        nseq = vh / sm.H;
        h = vh % sm.H;
    } else {
        const int npw = MAP ? sm.NS - sm.N : sm.NS;  // workgroups per head
        const int wi = blockIdx.x % npw;
        h = blockIdx.x / npw;
        nseq = MAP ? sm.seq_of_inner<true>(wi) : sm.seq_of<true>(wi);
        seg = (MAP ? wi + nseq : wi) - sm.seg_base<true>(nseq);
    }
    const long slot = sm.slot<PACKED>(nseq, h) + seg;  // workspace slot
    const long row0 = h * sm.hs + sm.start<PACKED>(nseq); // first input row of the sequence
    const bf16_t* kh = k + row0 * DK;
    const bf16_t* qh = q + row0 * DK;
    const bf16_t* vh = v + row0 * NS;
    const bf16_t* bh = beta + row0;

    // this wave's state column tiles: slot j holds tile id w + 8j (if < NCT);
    // ids below NCN are columns of S (OUT, STATES) or N (MAP), the rest columns of M
    v4f X[SLOTS][XR];
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
        const int id = w + NWV * j;
        const bool is_m = id >= Y::NCN;
        const int col = 16 * (is_m ? id - Y::NCN : id) + li;
#pragma unroll
        for (int i = 0; i < XR; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * i + 4 * g + r;
                float x = 0.f;
                if (id < Y::NCT) {
                    if constexpr (!MAP) x = state_in[(slot * DK + row) * NS + col];
                    else x = (is_m && row == col) ? 1.f : 0.f;
                }
                X[j][i][r] = x;
            }
    }

    const int L = sm.L;
    const int t_end = min((seg + 1) * L, sm.length<PACKED>(nseq));
    // The next chunk's rows are loaded into registers while this one is
    // processed.  Buffer resources end at the segment end: rows past it read
    // as zero with no guard (a guard would make the load's result wanted at
    // once), so the loads stay in flight until the chunk is staged.
    const rsrc_t rk = make_rsrc(kh, (uint32_t)t_end * DK * 2);
    const rsrc_t rq = make_rsrc(qh, (uint32_t)t_end * DK * 2);
    const rsrc_t rv = make_rsrc(vh, (uint32_t)t_end * NS * 2);
    const rsrc_t rb = make_rsrc(bh, (uint32_t)t_end * 2);
    const rsrc_t ra = make_rsrc(GATED ? alpha + row0 : nullptr, GATED ? (uint32_t)t_end * 4 : 0u);
    ChunkRegs<bf16_t, DK, NT> kr, qr;
    ChunkRegs<bf16_t, NS, NT> vr;
    unsigned short bnext = 0;
    unsigned anext = 0;
    constexpr int RPT = (kRecPieces + NT - 1) / NT;  // 16-byte pieces of a T record per thread
    uint4 tnext[RPT];  // this thread's pieces of the chunk's T record
    auto load_chunk = [&](int c, int tid) {
        // the output pass reads its rows for the last time: non-temporal
        constexpr int CP = OUT ? kLastUse : 0;
        kr.template load_buf<CP>(rk, c, tid);
        if constexpr (OUT) qr.template load_buf<CP>(rq, c, tid);
        vr.template load_buf<CP>(rv, c, tid);
        const long rec = sm.chunk_rec<PACKED>(nseq, h, c / CH, CH) * kRecElems;
#pragma unroll
        for (int e = 0; e < RPT; ++e)  // kRecPieces x 16 bytes: one record
            if (NT * (e + 1) <= kRecPieces || tid + NT * e < kRecPieces)
                tnext[e] = *reinterpret_cast<const uint4*>(trec + rec + (tid + NT * e) * 8);
        if (tid < CH) {
            bnext = __builtin_amdgcn_raw_buffer_load_b16(rb, (uint32_t)(c + tid) * 2, 0, 0);
            if constexpr (GATED) anext = __builtin_amdgcn_raw_buffer_load_b32(ra, (uint32_t)(c + tid) * 4, 0, 0);
        }
    };
    load_chunk(seg * L, tid);
    // Upper blocks of P (keys after every query of the tile) and of T are
    // read as zero operands and never written: clear them once.
    dchunk::clear_upper<RowLayout<LT, true>>(Ts, tid);
    if constexpr (OUT) {
        for (int e = tid; e < 6 * 256; e += NT) {
            const int tile = e >> 8, r = (e >> 4) & 15, c = e & 15;
            const int bi = tile < 3 ? 0 : tile < 5 ? 1 : 2;
            const int bj = tile < 3 ? tile + 1 : tile < 5 ? tile - 1 : 3;
            Ps[(16 * bi + r) * LT + pcol(16 * bj + c)] = M::cvt(0.f);
        }
    }
    for (int c0 = seg * L; c0 < t_end; c0 += CH) {
        // Gated: the lane indices are re-derived from an opaque copy every
        // chunk.  Otherwise the many per-lane LDS addresses built from them
        // are hoisted out of the loop and held, then spilled, for its whole
        // length; recomputed here they live only next to their uses.  (The
        // ungated eight-wave kernels fit with hoisted addresses and run
        // faster so; sixteen-wave ones have half the registers.)
        int tid_v = threadIdx.x;
        if constexpr (GATED || NWV == 16) asm volatile("" : "+v"(tid_v));
        const int tid = tid_v, lane = tid & 63, g = lane >> 4, li = lane & 15;
        const int n = min(CH, t_end - c0);
        // the state entering this chunk, as bf16 tiles: the state pass, and the
        // output pass of a training forward (uniform batches) when given
        if (MODE == kStates || (OUT && !PACKED && states != nullptr)) {
            const long ci = ((long)nseq * sm.H + h) * ((sm.T + CH - 1) / CH) + c0 / CH;
#pragma unroll
            for (int j = 0; j < SLOTS; ++j) {
                const int id = w + NWV * j;
                if (id >= Y::NCN) continue;
#pragma unroll
                for (int i = 0; i < XR; ++i) dchunk::put_tile(states + dchunk::tile_offset<DK, NS>(ci, id, i, lane), X[j][i]);
            }
        }
        // ---- stage the chunk row-major (transposed operands are read with
        // transpose loads)
        if (flags & kNormQK) {
            stage_rows_l2<DK, NT>(kr, tid, Ks, LQ);
            if constexpr (!MAP) stage_rows_l2<DK, NT, false, true>(kr, tid, Kf, LQ);
            if constexpr (OUT) stage_rows_l2<DK, NT, false, true>(qr, tid, Qs, Y::LW);
        } else {
            stage_rows_raw<bf16_t, DK, NT>(kr, tid, Ks, LQ);
            if constexpr (!MAP) stage_rows_raw<bf16_t, DK, NT, false, true>(kr, tid, Kf, LQ);
            if constexpr (OUT) stage_rows_raw<bf16_t, DK, NT, false, true>(qr, tid, Qs, Y::LW);
        }
        stage_rows_raw<bf16_t, NS, NT>(vr, tid, Vs, LV);
#pragma unroll
        for (int e = 0; e < RPT; ++e) {
            const int p = tid + NT * e;
            if (NT * (e + 1) <= kRecPieces || p < kRecPieces) {
                int row, col;
                dchunk::rec_piece(p, row, col);
                __bf16* dt = &Ts[row * LT];  // permuted rows
                *reinterpret_cast<uint2*>(dt + pcol(col)) = make_uint2(tnext[e].x, tnext[e].y);
                *reinterpret_cast<uint2*>(dt + pcol(col + 4)) = make_uint2(tnext[e].z, tnext[e].w);
            }
        }
        if (tid < CH) {  // wave 0
            const float braw = bf16_to_f32(bnext);
            Bs[tid] = (flags & kBetaSigmoid) ? 1.f / (1.f + __expf(-braw)) : braw;
            if constexpr (GATED) {
                // inclusive scan of the log-gates over the chunk; tokens past
                // the segment end count as alpha = 1, so gamma_C = gamma_{n-1}
                float lg = tid < n ? fmaxf(logf(__uint_as_float(anext)), -20.f) : 0.f;
#pragma unroll
                for (int off = 1; off < CH; off <<= 1) {
                    const float y = __shfl_up(lg, off);
                    lg += lane >= off ? y : 0.f;
                }
                const float lend = __shfl(lg, CH - 1);
                Gl[tid] = lg;
                Ge[tid] = expf(lg);
                Gc[tid] = expf(lend - lg);
            }
        }
        if (c0 + CH < t_end) load_chunk(c0 + CH, tid);
        __syncthreads();

        // ---- outputs: the causal scores P = tril(Q K^T) (bf16, rows =
        // queries; gated: o Gamma), computed as transposed tiles so each lane
        // writes four consecutive keys; wave w builds lower tiles w, w + 8;
        // then O^T = S^T Q^T with the state entering the chunk
        v4f Oq[OUT ? 4 : 1];
        if constexpr (OUT) {
#pragma unroll
            for (int jj = 0; jj < (10 + NWV - 1) / NWV; ++jj) {
                const int id = w + NWV * jj;
                if (id >= 10) break;
                int bi, bj;
                lower_tile(id, bi, bj);
                v4f acc = zero4();
#pragma unroll
                for (int kb = 0; kb < DK / 32; ++kb)
                    M::mma(acc, M::load_p(&Kf[(16 * bj + li) * LQ + 32 * kb], g),
                           M::load_p(&Qs[(16 * bi + li) * Y::LW + 32 * kb], g));
                if constexpr (GATED) {  // gamma_query / gamma_key
                    const float gq = Gl[16 * bi + li];
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[r] *= __expf(gq - Gl[16 * bj + 4 * g + r]);
                }
                uint2 pk;
                pk.x = pack_bf16x2((bi == bj && 4 * g + 0 > li) ? 0.f : acc[0],
                                   (bi == bj && 4 * g + 1 > li) ? 0.f : acc[1]);
                pk.y = pack_bf16x2((bi == bj && 4 * g + 2 > li) ? 0.f : acc[2],
                                   (bi == bj && 4 * g + 3 > li) ? 0.f : acc[3]);
                *reinterpret_cast<uint2*>(&Ps[(16 * bi + li) * LT + pcol(16 * bj + 4 * g)]) = pk;
            }
#pragma unroll
            for (int qt = 0; qt < 4; ++qt) {
                Oq[qt] = zero4();
                if (w < Y::NCT) {
#pragma unroll
                    for (int kb = 0; kb < DK / 32; ++kb)
                        M::mma(Oq[qt], M::from_tiles(X[0][2 * kb], X[0][2 * kb + 1]),
                               M::load_p(&Qs[(16 * qt + li) * Y::LW + 32 * kb], g));
                }
                if constexpr (GATED) Oq[qt] *= Ge[16 * qt + li];  // diag(gamma) Q S
            }
        }

        v4f U[SLOTS][4];
        if constexpr (MAP) {
            // ---- the map pass (sixteen waves at d = 128, each with one
            // tile): W = T K (gated: T diag(gamma) K, gamma applied to the T
            // fragment's columns in registers) is built once by all waves as
            // transposed tiles (rows land as 8-byte stores), with this wave's
            // U_v = T V columns; then U = U_v - W S
#pragma unroll
            for (int c = 0; c < Y::W_TPW; ++c) {
                const int dkt = w % XR, tt = (w / XR) * Y::W_TPW + c;
                v4f acc = zero4();
#pragma unroll
                for (int kb = 0; kb < CH / 32; ++kb) {
                    if (32 * kb > 16 * tt + 15) continue;  // T is lower triangular
                    frag tf = M::load_p(&Ts[(16 * tt + li) * LT + 32 * kb], g);
                    if constexpr (GATED) {  // slot s <-> column 32 kb + 4g + s (s < 4), 32 kb + 16 + 4g + s - 4
                        const v4f g0 = *reinterpret_cast<const v4f*>(&Ge[32 * kb + 4 * g]);
                        const v4f g1 = *reinterpret_cast<const v4f*>(&Ge[32 * kb + 16 + 4 * g]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            tf[e] = M::cvt((float)tf[e] * g0[e]);
                            tf[4 + e] = M::cvt((float)tf[4 + e] * g1[e]);
                        }
                    }
                    M::mma(acc, M::load_tr(Ks, LQ, 32 * kb, 16 * dkt, lane), tf);
                }
                __bf16* dst = &Ws[(16 * tt + li) * Y::LW + pcol(16 * dkt + 4 * g)];
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[r] = M::cvt(acc[r]);
            }
#pragma unroll
            for (int j = 0; j < SLOTS; ++j) {
                const int id = w + NWV * j;
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    U[j][tt] = zero4();
                    if (id < Y::NCN) {
#pragma unroll
                        for (int kb = 0; kb < CH / 32; ++kb) {
                            if (32 * kb > 16 * tt + 15) continue;
                            M::mma(U[j][tt], M::load_p(&Ts[(16 * tt + li) * LT + 32 * kb], g),
                                   M::load_tr(Vs, LV, 32 * kb, 16 * id, lane));
                        }
                    }
                }
            }
            __syncthreads();
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                v4f ws_[SLOTS];
#pragma unroll
                for (int j = 0; j < SLOTS; ++j) ws_[j] = zero4();
#pragma unroll
                for (int kb = 0; kb < DK / 32; ++kb) {
                    const frag wf = M::load_p(&Ws[(16 * tt + li) * Y::LW + 32 * kb], g);
#pragma unroll
                    for (int j = 0; j < SLOTS; ++j)
                        if (w + NWV * j < Y::NCT) M::mma(ws_[j], wf, M::from_tiles(X[j][2 * kb], X[j][2 * kb + 1]));
                }
#pragma unroll
                for (int j = 0; j < SLOTS; ++j) U[j][tt] -= ws_[j];
            }
        } else {
            // ---- output and state passes: U = T (V - diag(gamma) K S) per
            // column tile, without W (measured faster at eight waves, slower
            // for the sixteen-wave map pass)
            // ---- this wave's corrections U = T (V - diag(gamma) K S), per column
            // tile: R = V - diag(gamma) K S (K rows from LDS, S from registers),
            // then U = T R.  Every K and T fragment is read once for all of the
            // wave's tiles; the state-free W = T K never goes through LDS.
            {
                v4f ks[SLOTS][4];
#pragma unroll
                for (int j = 0; j < SLOTS; ++j)
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) ks[j][tt] = zero4();
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                    for (int kb = 0; kb < DK / 32; ++kb) {
                        const frag kf = M::load_p(&Kf[(16 * tt + li) * LQ + 32 * kb], g);
#pragma unroll
                        for (int j = 0; j < SLOTS; ++j)
                            if (w + NWV * j < Y::NCT) M::mma(ks[j][tt], kf, M::from_tiles(X[j][2 * kb], X[j][2 * kb + 1]));
                    }
                frag rf[SLOTS][CH / 32];  // R as B operands (the slot order of from_tiles and load_tr)
#pragma unroll
                for (int j = 0; j < SLOTS; ++j) {
                    const int id = w + NWV * j;
#pragma unroll
                    for (int kb = 0; kb < CH / 32; ++kb) {
                        frag vf = M::zero();
                        if (id < Y::NCN) vf = M::load_tr(Vs, LV, 32 * kb, 16 * id, lane);  // M columns: no values
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int h = e >> 2, r = e & 3, t = 32 * kb + 16 * h + 4 * g + r;
                            rf[j][kb][e] = M::cvt((float)vf[e] - (GATED ? Ge[t] : 1.f) * ks[j][2 * kb + h][r]);
                        }
                    }
                }
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
                    for (int j = 0; j < SLOTS; ++j) U[j][tt] = zero4();
#pragma unroll
                    for (int kb = 0; kb < CH / 32; ++kb) {
                        if (32 * kb > 16 * tt + 15) continue;  // T is lower triangular
                        const frag tf = M::load_p(&Ts[(16 * tt + li) * LT + 32 * kb], g);
#pragma unroll
                        for (int j = 0; j < SLOTS; ++j)
                            if (w + NWV * j < Y::NCT) M::mma(U[j][tt], tf, rf[j][kb]);
                    }
                }
            }
        }
        if constexpr (OUT) __syncthreads();  // P of every wave

        // ---- the state chain over this wave's column tiles.  The chain is
        // bound by LDS reads, so every operand fragment (a transposed row
        // block of K, a row block of P) is read once and applied to all of
        // the wave's tiles.
        // beta o U (and, if wanted, the predictions V - U)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
            for (int j = 0; j < SLOTS; ++j) {
                const int id = w + NWV * j;
                if (id >= Y::NCT) continue;
                if constexpr (OUT) {
                    if (pred) {  // rows past the segment end are dropped by the resource
                        const rsrc_t rp = make_rsrc(pred + row0 * NS, (uint32_t)t_end * NS * 2);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int t = 16 * tt + 4 * g + r;
                            const float pv = (float)Vs[t * LV + 16 * id + li] - U[j][tt][r];
                            __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(pv), rp,
                                                                  (uint32_t)(((c0 + t) * NS + 16 * id + li) * 2), 0, 0);
                        }
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) U[j][tt][r] *= Bs[16 * tt + 4 * g + r];
            }
        }
#pragma unroll
        for (int j = 0; j < SLOTS; ++j) {
            const int id = w + NWV * j;
            if (id >= Y::NCT) continue;
            if constexpr (OUT) {
                // outputs, second half: O^T += (beta o U)^T P^T, stored
                bf16_t* oh = o + (row0 + c0) * NS + 16 * id + 4 * g;
#pragma unroll
                for (int qt = 0; qt < 4; ++qt) {
#pragma unroll
                    for (int kb = 0; kb < CH / 32; ++kb) {
                        if (32 * kb > 16 * qt + 15) continue;  // keys after these queries
                        M::mma(Oq[qt], M::from_tiles(U[j][2 * kb], U[j][2 * kb + 1]),
                               M::load_p(&Ps[(16 * qt + li) * LT + 32 * kb], g));
                    }
                    const int t = 16 * qt + li;
                    if (t < n) {
                        uint2 pk;
                        pk.x = pack_bf16x2(Oq[qt][0], Oq[qt][1]);
                        pk.y = pack_bf16x2(Oq[qt][2], Oq[qt][3]);
                        *reinterpret_cast<uint2*>(oh + (long)t * NS) = pk;
                    }
                }
            }
            // gated: S = gamma_C S + K^T (beta gamma_C / gamma o U)
            if constexpr (GATED) {
                const float gend = Ge[CH - 1];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) U[j][tt][r] *= Gc[16 * tt + 4 * g + r];
#pragma unroll
                for (int i = 0; i < XR; ++i) X[j][i] *= gend;
            }
        }
        // S += K^T (beta o U)
#pragma unroll
        for (int i = 0; i < XR; ++i)
#pragma unroll
            for (int kb = 0; kb < CH / 32; ++kb) {
                const frag kf = M::load_tr(Ks, LQ, 32 * kb, 16 * i, lane);
#pragma unroll
                for (int j = 0; j < SLOTS; ++j)
                    if (w + NWV * j < Y::NCT) M::mma(X[j][i], kf, M::from_tiles(U[j][2 * kb], U[j][2 * kb + 1]));
            }
        __syncthreads();
    }

    // ---- the segment's result: S_T (OUT, last segment) or the maps (MAP)
    if constexpr (MODE == kStates) return;
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
        const int id = w + NWV * j;
        if (id >= Y::NCT) continue;
        const bool is_m = id >= Y::NCN;
        float* dst;
        int ld, col;
        if constexpr (OUT) {
            if (seg != sm.segs<PACKED>(nseq) - 1 || !S_out) continue;
            dst = S_out + ((long)nseq * sm.H + h) * DK * NS;
            ld = NS;
            col = 16 * id + li;
        } else {
            dst = is_m ? map_m + slot * DK * DK : map_n + slot * DK * NS;
            ld = is_m ? DK : NS;
            col = 16 * (is_m ? id - Y::NCN : id) + li;
        }
#pragma unroll
        for (int i = 0; i < XR; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(16 * i + 4 * g + r) * ld + col] = X[j][i][r];
    }
}

// Waves per workgroup of the map pass: with dk = dv = 128 it carries 16
// state column tiles, one per wave of a sixteen-wave workgroup (twice the
// waves per SIMD to hide LDS-operand latency, half the registers per wave).
template <int DK, int DV>
constexpr int kMapWaves = (DK == 128 && DV == 128) ? 16 : 8;
// Waves per workgroup of the output pass.
template <int DK, int DV>
constexpr int kOutWaves = 8;

// XCDs of the chip: dispatch places block b on XCD b mod 8.
constexpr int kXcds = 8;

// Blocks of delta_compose_kernel for NH states.
template <int DV>
inline unsigned compose_blocks(int NH) { return (unsigned)(((NH + kXcds - 1) / kXcds) * kXcds * (DV / 16)); }

// S_in(0) = S0 (or 0); S_in(g+1) = M_g S_in(g) + N_g in fp32 MFMA.  One
// workgroup per (16-column block of the state, sequence and head); serial
// over the sequence's segments.  REV runs the transposed recurrence from the
// last segment down (the backward pass: G(G-1) = S0, G(g-1) = M_g^T G(g) +
// N_g, with M_g the forward's segment map as stored).
// Every column block of a head reads the whole of each M_g, so the blocks of
// one head are numbered to land on one XCD (dispatch places block b on XCD
// b mod 8, and each XCD has its own L2): M_g then comes from memory once per
// head instead of once per column block.  M_g is staged in LDS, and M_{g+1},
// N_{g+1} are loaded into registers while step g runs; the staged rows are
// DK + 4 floats apart, so the 16-byte row reads of each eight consecutive
// lanes fall in distinct banks.
template <int DK, int DV, bool PACKED, bool REV = false>
__global__ __launch_bounds__(256) void delta_compose_kernel(const float* __restrict__ map_n,
                                                            const float* __restrict__ map_m,
                                                            const float* S0, float* __restrict__ state_in,
                                                            SegMap sm) {
    constexpr int RPW = DK / 64;              // row tiles per wave
    constexpr int LM = DK + 4;                // row stride of the staged map
    constexpr int MV = DK * DK / (4 * 256);   // 16-byte pieces of a map per thread
    __shared__ float Sb[DK][17];
    __shared__ __align__(16) float Ms[DK * LM];
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, li = lane & 15;
    const int w = wave_id(tid);
    __builtin_assume(w >= 0 && w < 4);  // four waves
    // block b = (p / 8) (8 NCB) + ct 8 + p % 8
    constexpr int NCB = DV / 16;
    const int b = blockIdx.x, xcd = b % kXcds, rest = b / kXcds;
    const int ct = rest % NCB, col = 16 * ct + li;
    const int p = (rest / NCB) * kXcds + xcd;  // the state's index in S0
    if (p >= sm.N * sm.H) return;
    const int nseq = p / sm.H, h = p % sm.H;
    const long base = sm.slot<PACKED>(nseq, h);  // slot of the sequence's first segment
    int G = sm.segs<PACKED>(nseq);
    G = G < 0 ? 0 : (G > sm.NS - sm.seg_base<PACKED>(nseq) ? sm.NS - sm.seg_base<PACKED>(nseq) : G);
    if (G == 0) return;
    auto map_of = [&](int s) -> long { return REV ? base + G - 1 - s : base + s; };  // the map of step s
    v4f mreg[MV];
    v4f nreg[RPW];
    auto load_map = [&](long from) {
        const float* Mg = map_m + from * DK * DK;
        const float* Ng = map_n + from * DK * DV;
#pragma unroll
        for (int j = 0; j < MV; ++j) mreg[j] = *reinterpret_cast<const v4f*>(Mg + 4 * (j * 256 + tid));
#pragma unroll
        for (int i = 0; i < RPW; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) nreg[i][r] = Ng[(16 * (w * RPW + i) + 4 * g + r) * DV + col];
    };
    // The initial state: every load issued before the first store (a load
    // behind a store would wait for that store, as both count in vmcnt).
    v4f acc[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) acc[i] = zero4();
    if (S0) {
#pragma unroll
        for (int i = 0; i < RPW; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][r] = S0[((long)p * DK + 16 * (w * RPW + i) + 4 * g + r) * DV + col];
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int rt = w * RPW + i;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * rt + 4 * g + r;
            Sb[row][li] = acc[i][r];
            state_in[((REV ? base + G - 1 : base) * DK + row) * DV + col] = acc[i][r];
        }
    }
    if (G > 1) load_map(map_of(0));
    for (int s = 0; s + 1 < G; ++s) {
        const long to = REV ? map_of(s) - 1 : map_of(s) + 1;  // the state step s produces
#pragma unroll
        for (int j = 0; j < MV; ++j) {
            const int e = 4 * (j * 256 + tid), row = e / DK, c = e % DK;
            *reinterpret_cast<v4f*>(&Ms[row * LM + c]) = mreg[j];
        }
#pragma unroll
        for (int i = 0; i < RPW; ++i) acc[i] = nreg[i];
        __syncthreads();  // Ms and Sb written
        if (s + 2 < G) load_map(map_of(s + 1));
#pragma unroll 4
        for (int kb = 0; kb < DK / 16; ++kb) {
            v4f bb;
#pragma unroll
            for (int e = 0; e < 4; ++e) bb[e] = Sb[16 * kb + 4 * g + e][li];
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                const int rt = w * RPW + i;
                v4f a;
                if constexpr (REV) {  // (M^T)[16 rt + li][16 kb + 4 g + e]: lane groups g hit distinct banks
#pragma unroll
                    for (int e = 0; e < 4; ++e) a[e] = Ms[(16 * kb + 4 * g + e) * LM + 16 * rt + li];
                } else {
                    a = *reinterpret_cast<const v4f*>(&Ms[(16 * rt + li) * LM + 16 * kb + 4 * g]);
                }
                Mma<float>::mma(acc[i], a, bb);
            }
        }
        __syncthreads();  // every read of Ms and Sb done
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int rt = w * RPW + i;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * rt + 4 * g + r;
                Sb[row][li] = acc[i][r];
                state_in[(to * DK + row) * DV + col] = acc[i][r];
            }
        }
    }
}

// states (uniform batches only; NULL otherwise): a training forward, which
// also leaves the backward pass's context in ws -- the maps of every segment
// (the last one's M_g too) and every chunk's entering state as bf16 tiles in
// `states`.
template <int DK, int DV, bool GATED, bool PACKED>
hipError_t launch_packing(const bf16_t* q, const bf16_t* k, const bf16_t* v, const bf16_t* beta,
                        const float* alpha, const float* S0, bf16_t* o, float* S_out, bf16_t* pred, int flags,
                        const SegMap& sm, float* ws, hipStream_t stream, bf16_t* states = nullptr) {
    const size_t slots = (size_t)sm.H * sm.NS;
    float* map_n = ws;
    float* map_m = map_n + slots * DK * DV;
    float* state_in = map_m + slots * DK * DK;
    bf16_t* trec = reinterpret_cast<bf16_t*>(state_in + slots * DK * DV);
    const long recs = (long)sm.H * sm.chunk_recs_per_head(CH);
    hipError_t err;
    delta_tinv_kernel<DK, GATED, PACKED><<<dim3(recs), dim3(NT), 0, stream>>>(k, beta, alpha, trec, flags, sm);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const bool train = !PACKED && states != nullptr;
    if (sm.NS > sm.N) {  // training: every segment's map (M_g of the last for the backward's reverse composition)
        constexpr int NWM = kMapWaves<DK, DV>;
        const int maps = train ? sm.H * sm.NS : sm.H * (sm.NS - sm.N);
        delta_chunk_kernel<DK, DV, kMap, GATED, PACKED, NWM><<<dim3(maps), dim3(NWM * 64), 0, stream>>>(
            q, k, v, beta, alpha, nullptr, nullptr, map_n, map_m, nullptr, nullptr, nullptr, trec, flags, sm);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    delta_compose_kernel<DK, DV, PACKED><<<dim3(compose_blocks<DV>(sm.N * sm.H)), dim3(256), 0, stream>>>(
        map_n, map_m, S0, state_in, sm);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    constexpr int NWO = kOutWaves<DK, DV>;
    delta_chunk_kernel<DK, DV, kOut, GATED, PACKED, NWO><<<dim3(sm.H * sm.NS), dim3(NWO * 64), 0, stream>>>(
        q, k, v, beta, alpha, o, state_in, nullptr, nullptr, S_out, pred, train ? states : nullptr, trec, flags, sm);
    return hipGetLastError();
}

// The backward pass's forward sweep (uniform batches): maps, composition,
// then every chunk's entering state as bf16 tiles.
template <int DK, int DV, bool GATED>
hipError_t launch_states(const bf16_t* q, const bf16_t* k, const bf16_t* v, const bf16_t* beta, const float* alpha,
                         const float* S0, bf16_t* states, const SegMap& sm, float* ws, hipStream_t stream) {
    const size_t slots = (size_t)sm.H * sm.NS;
    float* map_n = ws;
    float* map_m = map_n + slots * DK * DV;
    float* state_in = map_m + slots * DK * DK;
    bf16_t* trec = reinterpret_cast<bf16_t*>(state_in + slots * DK * DV);
    const long recs = (long)sm.H * sm.chunk_recs_per_head(CH);
    hipError_t err;
    delta_tinv_kernel<DK, GATED, false><<<dim3(recs), dim3(NT), 0, stream>>>(k, beta, alpha, trec, 0, sm);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (sm.G > 1) {  // every segment's map: M_0..M_{G-2} for the composition below, M_1..M_{G-1} for the backward's
        constexpr int NWM = kMapWaves<DK, DV>;
        delta_chunk_kernel<DK, DV, kMap, GATED, false, NWM><<<dim3(sm.H * sm.NS), dim3(NWM * 64), 0, stream>>>(
            q, k, v, beta, alpha, nullptr, nullptr, map_n, map_m, nullptr, nullptr, nullptr, trec, 0, sm);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    delta_compose_kernel<DK, DV, false><<<dim3(compose_blocks<DV>(sm.N * sm.H)), dim3(256), 0, stream>>>(
        map_n, map_m, S0, state_in, sm);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    delta_chunk_kernel<DK, DV, kStates, GATED, false><<<dim3(sm.H * sm.NS), dim3(NT), 0, stream>>>(
        q, k, v, beta, alpha, nullptr, state_in, nullptr, nullptr, nullptr, nullptr, states, trec, 0, sm);
    return hipGetLastError();
}

template <int DK, int DV, bool GATED>
hipError_t launch_typed(const bf16_t* q, const bf16_t* k, const bf16_t* v, const bf16_t* beta,
                        const float* alpha, const float* S0, bf16_t* o, float* S_out, bf16_t* pred, int flags,
                        const SegMap& sm, float* ws, hipStream_t stream) {
    return sm.packed()
               ? launch_packing<DK, DV, GATED, true>(q, k, v, beta, alpha, S0, o, S_out, pred, flags, sm, ws, stream)
               : launch_packing<DK, DV, GATED, false>(q, k, v, beta, alpha, S0, o, S_out, pred, flags, sm, ws, stream);
}

template <int DK, int DV>
hipError_t launch_train(const bf16_t* q, const bf16_t* k, const bf16_t* v, const bf16_t* beta, const float* alpha,
                        const float* S0, bf16_t* o, float* S_out, const SegMap& sm, float* ws, bf16_t* states,
                        hipStream_t stream) {
    return alpha ? launch_packing<DK, DV, true, false>(q, k, v, beta, alpha, S0, o, S_out, nullptr, 0, sm, ws, stream,
                                                       states)
                 : launch_packing<DK, DV, false, false>(q, k, v, beta, nullptr, S0, o, S_out, nullptr, 0, sm, ws,
                                                        stream, states);
}

}  // namespace

hipError_t launch_delta_forward_train(const void* q, const void* k, const void* v, const void* beta,
                                      const float* alpha, const float* S0, void* o, float* S_out, void* states,
                                      const SegMap& sm, int dk, int dv, float* ws, hipStream_t stream) {
    if (sm.packed() || !states) return hipErrorInvalidValue;
    const bf16_t* qb = static_cast<const bf16_t*>(q);
    const bf16_t* kb = static_cast<const bf16_t*>(k);
    const bf16_t* vb = static_cast<const bf16_t*>(v);
    const bf16_t* bb = static_cast<const bf16_t*>(beta);
    bf16_t* ob = static_cast<bf16_t*>(o);
    bf16_t* st = static_cast<bf16_t*>(states);
#define TRAIN_CASE(A, B) \
    if (dk == A && dv == B) return launch_train<A, B>(qb, kb, vb, bb, alpha, S0, ob, S_out, sm, ws, st, stream);
    TRAIN_CASE(64, 64)
    TRAIN_CASE(64, 128)
    TRAIN_CASE(128, 64)
    TRAIN_CASE(128, 128)
#undef TRAIN_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_delta_states(const void* q, const void* k, const void* v, const void* beta, const float* alpha,
                               const float* S0, void* states, const SegMap& sm, int dk, int dv, float* ws,
                               hipStream_t stream) {
    const bf16_t* qb = static_cast<const bf16_t*>(q);
    const bf16_t* kb = static_cast<const bf16_t*>(k);
    const bf16_t* vb = static_cast<const bf16_t*>(v);
    const bf16_t* bb = static_cast<const bf16_t*>(beta);
    bf16_t* st = static_cast<bf16_t*>(states);
    if (sm.packed()) return hipErrorInvalidValue;
#define STATES_CASE(A, B)                                                                         \
    if (dk == A && dv == B)                                                                       \
        return alpha ? launch_states<A, B, true>(qb, kb, vb, bb, alpha, S0, st, sm, ws, stream)   \
                     : launch_states<A, B, false>(qb, kb, vb, bb, nullptr, S0, st, sm, ws, stream);
    STATES_CASE(64, 64)
    STATES_CASE(64, 128)
    STATES_CASE(128, 64)
    STATES_CASE(128, 128)
#undef STATES_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_delta_compose(const float* map_n, const float* map_m, const float* S0, float* state_in,
                                const SegMap& sm, int dk, int dv, hipStream_t stream) {
    if (sm.packed()) return hipErrorInvalidValue;
#define FWD_CASE(A, B)                                                                                        \
    if (dk == A && dv == B) {                                                                                 \
        delta_compose_kernel<A, B, false><<<dim3(compose_blocks<B>(sm.N * sm.H)), dim3(256), 0, stream>>>(   \
            map_n, map_m, S0, state_in, sm);                                                                  \
        return hipGetLastError();                                                                             \
    }
    FWD_CASE(64, 64)
    FWD_CASE(64, 128)
    FWD_CASE(128, 64)
    FWD_CASE(128, 128)
#undef FWD_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_delta_compose_rev(const float* map_c, const float* map_mt, const float* G_last, float* g_end,
                                    const SegMap& sm, int dk, int dv, hipStream_t stream) {
    if (sm.packed()) return hipErrorInvalidValue;
#define REV_CASE(A, B)                                                                                        \
    if (dk == A && dv == B) {                                                                                 \
        delta_compose_kernel<A, B, false, true><<<dim3(compose_blocks<B>(sm.N * sm.H)), dim3(256), 0, stream>>>(        \
            map_c, map_mt, G_last, g_end, sm);                                                                \
        return hipGetLastError();                                                                             \
    }
    REV_CASE(64, 64)
    REV_CASE(64, 128)
    REV_CASE(128, 64)
    REV_CASE(128, 128)
#undef REV_CASE
    return hipErrorInvalidValue;
}

size_t delta_ws_floats(long slots, long recs, int dk, int dv) {
    // per slot: N_g, M_g, S_in; per chunk record: T (bf16, two per float)
    return (size_t)slots * ((size_t)dk * dv + (size_t)dk * dk + (size_t)dk * dv) + (size_t)recs * kRecElems / 2;
}

hipError_t launch_delta_forward(const void* q, const void* k, const void* v, const void* beta,
                                const float* alpha, const float* S0, void* o, float* S_out, void* pred, int flags,
                                const SegMap& sm, int dk, int dv, int dtype, float* ws, hipStream_t stream) {
    if (dtype != 1) return hipErrorInvalidValue;
    const bf16_t* qb = static_cast<const bf16_t*>(q);
    const bf16_t* kb = static_cast<const bf16_t*>(k);
    const bf16_t* vb = static_cast<const bf16_t*>(v);
    const bf16_t* bb = static_cast<const bf16_t*>(beta);
    bf16_t* ob = static_cast<bf16_t*>(o);
    bf16_t* pb = static_cast<bf16_t*>(pred);
#define DELTA_CASE(A, B)                                                                                      \
    if (dk == A && dv == B)                                                                                   \
        return alpha ? launch_typed<A, B, true>(qb, kb, vb, bb, alpha, S0, ob, S_out, pb, flags, sm, ws, stream)   \
                     : launch_typed<A, B, false>(qb, kb, vb, bb, nullptr, S0, ob, S_out, pb, flags, sm, ws, stream);
    DELTA_CASE(64, 64)
    DELTA_CASE(64, 128)
    DELTA_CASE(128, 64)
    DELTA_CASE(128, 128)
#undef DELTA_CASE
    return hipErrorInvalidValue;
}

}  // namespace la
