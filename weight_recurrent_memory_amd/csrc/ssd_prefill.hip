// Scalar-decay linear memory (the Mamba-2 / SSD form), chunked prefill on gfx950.
//
// The rule ("线性注意力与 SSM:两条技术路线的完整推导" §3, the Mamba-2 paragraph:
// the outer-product state of linear attention with a scalar decay on the old
// state; written key-first):
//   S_t = alpha_t S_{t-1} + k_t v_t^T,     o_t = S_t^T q_t   (write, then read).
// With d = 1 it is the selective scan of "手撕：递推与记忆模型"; its explicit
// mixing matrix weighs input i in output j by c_j b_i prod_{i<s<=j} a_s.
//
// Chunked form.  Over a chunk of C = 64 tokens entered with state S, with the
// chunk-local products gamma_t = alpha_{c0} ... alpha_t:
//   O   = diag(gamma) Q S + (tril(Q K^T) o Gamma) V,   Gamma[t][i] = gamma_t / gamma_i,
//   S' = gamma_C S + K^T diag(gamma_C / gamma) V.
// Every ratio is 2^(difference of chunk-local prefix sums of log2 alpha); each
// log is clamped at log2(e^-20), so no ratio divides by an underflowed
// product.  Each wave rebuilds the chunk's prefix sums in its own 64 lanes
// (lane = token) from one gate per lane, so a decay factor anywhere in the
// chunk is a lane shuffle away.
//
// Sequence parallelism.  A segment maps its incoming state affinely with a
// scalar: S_out = 2^(l_g) S_in + N_g, l_g the segment's sum of log2 alpha and
// N_g the segment run from a zero state.  Three launches:
//   ssd_segment_kernel   (N_g, l_g) for every segment but the last
//   ssd_compose_kernel   S_in(g+1) = 2^(l_g) S_in(g) + N_g, elementwise, serial in g
//   ssd_output_kernel    the chunk loop from S_in(g), writing O (and S_T last)
#include "common.hpp"
#include "kernels.hpp"

namespace la {

namespace {

constexpr int CH = kChunk;
constexpr int NTHR = 256;                              // four waves
constexpr float kLog2Floor = -28.853900817779268f;     // log2(e^-20)

template <int DK, int DV>
struct SL {
    static constexpr int LQ = DK + 8;         // bf16 rows with k = dk (K and S^T)
    static constexpr int LV = DV + 8;         // bf16 rows of V
    static constexpr int RTW = DK / 64;       // dk row tiles of the state per wave
    static constexpr int NVT = DV / 16;       // value column tiles
    static constexpr int KSZ = CH * LQ, VSZ = CH * LV, SSZ = DV * LQ;
    static constexpr int bytes(int nst) { return 2 * (2 * KSZ + 2 * VSZ + nst * SSZ); }
    // S^T double-buffered unless that costs a workgroup of residency.
    static constexpr int kLds = 160 * 1024;
    static constexpr int NST = (2 * bytes(2) <= kLds) ? 2 : (2 * bytes(1) <= kLds) ? 1 : (bytes(2) <= kLds) ? 2 : 1;
    static constexpr int LDS_BYTES = bytes(NST);
    static constexpr int SEG_BYTES = 2 * (2 * KSZ + 2 * VSZ);
};

// Inclusive prefix sum over the wave's lanes (lane = token of the chunk) of
// the clamped log2 gates; tokens at or past the segment end count as
// alpha = 1.  A NaN gate stays NaN.
__device__ __forceinline__ float log2_prefix(float a, bool valid, int lane) {
    const float l = log2f(a);
    float x = valid ? (l < kLog2Floor ? kLog2Floor : l) : 0.f;
#pragma unroll
    for (int off = 1; off < CH; off <<= 1) {
        const float y = __shfl_up(x, off);
        x += lane >= off ? y : 0.f;
    }
    return x;
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Chunk rows of K scaled per row by f(row) into LDS (bf16, row-major).  Every
// lane of the wave takes part (the row factors come through shuffles).
template <int D, typename F>
__device__ __forceinline__ void stage_rows_scaled(const ChunkRegs<bf16_t, D, NTHR>& cr, int tid, __bf16* rm,
                                                  int ld, F&& factor) {
    constexpr int NV = ChunkRegs<bf16_t, D, NTHR>::NV;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int row = ChunkRegs<bf16_t, D, NTHR>::row_of(j, tid);
        const int col = ChunkRegs<bf16_t, D, NTHR>::col_of(j, tid);
        const float f = factor(row);
        uint4 x;
        uint32_t* xs = reinterpret_cast<uint32_t*>(&x);
#pragma unroll
        for (int e = 0; e < 4; ++e) xs[e] = pack_bf16x2(cr.get(j, 2 * e) * f, cr.get(j, 2 * e + 1) * f);
        *reinterpret_cast<uint4*>(rm + row * ld + col) = x;
    }
}

// ------------------------------------------------------------- segment maps
//
// N_g = sum over the segment's chunks of (gamma_C-decayed) K^T diag(gamma_C /
// gamma) V, from a zero state; l_g = the segment's sum of log2 alpha.  Wave w
// owns dk rows 16 w RTW ..; the keys are staged already scaled by
// gamma_C / gamma_t.  NPF chunks are in flight ahead of the one staged.
template <int DK, int DV, bool PACKED>
__global__ __launch_bounds__(NTHR) void ssd_segment_kernel(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                                                           const float* __restrict__ alpha, float* __restrict__ map_n,
                                                           float* __restrict__ map_l, SegMap sm) {
    using LY = SL<DK, DV>;
    using M = Mma<bf16_t>;
    typedef M::frag frag;
    constexpr int RTW = LY::RTW, NVT = LY::NVT;
    constexpr int NPF = (DK + DV) * 2 <= 256 ? 4 : 2;
    __shared__ __align__(16) __bf16 lds[LY::SEG_BYTES / 2];
    __bf16* Kb = lds;
    __bf16* Vb = lds + 2 * LY::KSZ;

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, li = lane & 15;
    const int w = wave_id(tid);
    // (head, sequence, segment) of this workgroup: every segment but the
    // last of its sequence
    int h, nseq, seg;
    if constexpr (!PACKED) {  // (sequence, head)-major, segments consecutive
        const int vh = blockIdx.x / (sm.G - 1);
        seg = blockIdx.x % (sm.G - 1);
        nseq = vh / sm.H;
        h = vh % sm.H;
    } else {
        const int npw = sm.NS - sm.N;
        const int wi = blockIdx.x % npw;
        h = blockIdx.x / npw;
        nseq = sm.seq_of_inner<true>(wi);
        seg = wi + nseq - sm.seg_base<true>(nseq);
    }
    const long slot = sm.slot<PACKED>(nseq, h) + seg;
    const long row0 = h * sm.hs + sm.start<PACKED>(nseq);
    const int t0 = seg * sm.L, t1 = min(t0 + sm.L, sm.length<PACKED>(nseq));
    const rsrc_t rk = make_rsrc(k + row0 * DK, (uint32_t)t1 * DK * 2);
    const rsrc_t rv = make_rsrc(v + row0 * DV, (uint32_t)t1 * DV * 2);
    const rsrc_t ra = make_rsrc(alpha + row0, (uint32_t)t1 * 4);

    ChunkRegs<bf16_t, DK, NTHR> kr[NPF];
    ChunkRegs<bf16_t, DV, NTHR> vr[NPF];
    unsigned ar[NPF];
    auto load = [&](int p, int c) {
        kr[p].load_buf(rk, c, tid);
        vr[p].load_buf(rv, c, tid);
        ar[p] = __builtin_amdgcn_raw_buffer_load_b32(ra, (uint32_t)(c + lane) * 4, 0, 0);
    };
#pragma unroll
    for (int p = 0; p < NPF; ++p) load(p, t0 + p * CH);

    v4f acc[RTW][NVT];
#pragma unroll
    for (int i = 0; i < RTW; ++i)
#pragma unroll
        for (int c = 0; c < NVT; ++c) acc[i][c] = zero4();
    float lsum = 0.f;

    auto body = [&](auto slot, int c0) {
        constexpr int sl = decltype(slot)::value, b = sl & 1;
        __bf16* Ks = Kb + b * LY::KSZ;
        __bf16* Vs = Vb + b * LY::VSZ;
        const float lg = log2_prefix(__uint_as_float(ar[sl]), c0 + lane < t1, lane);
        const float lend = __shfl(lg, CH - 1);
        stage_rows_scaled<DK>(kr[sl], tid, Ks, LY::LQ, [&](int row) { return exp2_hw(lend - __shfl(lg, row)); });
        stage_rows_raw<bf16_t, DV, NTHR>(vr[sl], tid, Vs, LY::LV);
        load(sl, c0 + NPF * CH);
        __syncthreads();
        const float gC = exp2_hw(lend);
        lsum += lend;
#pragma unroll
        for (int i = 0; i < RTW; ++i)
#pragma unroll
            for (int c = 0; c < NVT; ++c) acc[i][c] *= gC;
#pragma unroll
        for (int j = 0; j < CH / 32; ++j)
#pragma unroll
            for (int i = 0; i < RTW; ++i) {
                const frag a = M::load_tr(Ks, LY::LQ, 32 * j, 16 * (w * RTW + i), lane);
#pragma unroll
                for (int c = 0; c < NVT; ++c) M::mma(acc[i][c], a, M::load_tr(Vs, LY::LV, 32 * j, 16 * c, lane));
            }
    };
    // Whole groups of NPF chunks with no exit inside: a chunk past the
    // segment end stages zero rows with gates of 1 and changes nothing.
    for (int c0 = t0; c0 < t1; c0 += NPF * CH) {
        body(std::integral_constant<int, 0>{}, c0);
        body(std::integral_constant<int, 1>{}, c0 + CH);
        if constexpr (NPF == 4) {
            body(std::integral_constant<int, 2>{}, c0 + 2 * CH);
            body(std::integral_constant<int, 3>{}, c0 + 3 * CH);
        }
    }

    float* dst = map_n + slot * DK * DV;
#pragma unroll
    for (int i = 0; i < RTW; ++i)
#pragma unroll
        for (int c = 0; c < NVT; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(16 * (w * RTW + i) + 4 * g + r) * DV + 16 * c + li] = acc[i][c][r];
    if (tid == 0) map_l[slot] = lsum;
}

// S_in(0) = S0 (or 0); S_in(g+1) = 2^(l_g) S_in(g) + N_g.  Elementwise: thread
// i of the grid owns four consecutive state elements of one (sequence, head)
// pair and walks that sequence's segments.  The
// segments are taken in batches whose loads are all issued before the first
// combine, so the serial chain costs one memory latency per batch.
template <int E, bool PACKED>
__global__ __launch_bounds__(256) void ssd_compose_kernel(const float* __restrict__ map_n,
                                                          const float* __restrict__ map_l, const float* S0,
                                                          float* __restrict__ state_in, SegMap sm) {
    constexpr int BATCH = 8;
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;  // 4-float group
    if (idx >= (long)sm.N * sm.H * (E / 4)) return;
    const int p = (int)(idx / (E / 4));  // the state's index in S0: sequence * H + head
    const int e = (int)(idx % (E / 4)) * 4;
    const int nseq = p / sm.H, h = p % sm.H;
    const long base = sm.slot<PACKED>(nseq, h);
    int G = sm.segs<PACKED>(nseq);
    G = G < 0 ? 0 : (G > sm.NS - sm.seg_base<PACKED>(nseq) ? sm.NS - sm.seg_base<PACKED>(nseq) : G);
    if (G == 0) return;
    const float* nh = map_n + base * E + e;
    const float* lh = map_l + base;
    float* sh = state_in + base * E + e;
    v4f s = S0 ? *reinterpret_cast<const v4f*>(S0 + (long)p * E + e) : zero4();
    *reinterpret_cast<v4f*>(sh) = s;
    for (int g0 = 0; g0 + 1 < G; g0 += BATCH) {
        v4f n[BATCH];
        float l[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u)
            if (g0 + u + 1 < G) {
                n[u] = *reinterpret_cast<const v4f*>(nh + (long)(g0 + u) * E);
                l[u] = lh[g0 + u];
            }
#pragma unroll
        for (int u = 0; u < BATCH; ++u)
            if (g0 + u + 1 < G) {
                s = exp2_hw(l[u]) * s + n[u];
                *reinterpret_cast<v4f*>(sh + (long)(g0 + u + 1) * E) = s;
            }
    }
}

// ------------------------------------------------------------- output pass
//
// Registers of one output-pass chunk in flight: K and V rows for the LDS
// staging, this wave's raw query fragments (rows 16w + lane % 16) and one
// gate per lane.
template <int DK, int DV>
struct SsdChunk {
    static constexpr int QF = DK / 32;
    ChunkRegs<bf16_t, DK, NTHR> kr;
    ChunkRegs<bf16_t, DV, NTHR> vr;
    v4u qraw[QF];
    unsigned araw;
    __device__ __forceinline__ void load(rsrc_t rq, rsrc_t rk, rsrc_t rv, rsrc_t ra, int c0, int w, int tid) {
        const int lane = tid & 63, g = lane >> 4, li = lane & 15;
        kr.load_buf(rk, c0, tid);
        vr.load_buf(rv, c0, tid);
#pragma unroll
        for (int kk = 0; kk < QF; ++kk)
            qraw[kk] = buf_load16(rq, (uint32_t)(((c0 + 16 * w + li) * DK + 32 * kk + 8 * g) * 2));
        araw = __builtin_amdgcn_raw_buffer_load_b32(ra, (uint32_t)(c0 + lane) * 4, 0, 0);
    }
};

// The chunk loop of wave W (a compile-time constant: straight-line body).
// Wave W owns query rows 16W..16W+15 of every chunk and dk rows 16 W RTW ..
// of the state.  Per chunk (state S entering it, lg the gate prefix sums):
//   P^T  = K Q_W^T o 2^(lg_query - lg_key), keys after the query zeroed
//   O_W^T = 2^(lg_query) S^T Q_W^T + V^T P^T        (stored from registers)
//   S    = 2^(lg_end) S + (K o 2^(lg_end - lg_key))^T V   (this wave's rows)
// K, V and the bf16 copy of S^T are shared through double-buffered LDS; the
// next chunk is staged while this one computes, one barrier per chunk.
template <int DK, int DV, int W>
__device__ __forceinline__ void ssd_output_pass(rsrc_t rq, rsrc_t rk, rsrc_t rv, rsrc_t ra, rsrc_t ro, int t_beg,
                                                int t_end, v4f (&S)[SL<DK, DV>::RTW][SL<DK, DV>::NVT],
                                                SsdChunk<DK, DV>& in, __bf16* lds, int tid) {
    using M = Mma<bf16_t>;
    typedef M::frag frag;
    using LY = SL<DK, DV>;
    constexpr int LQ = LY::LQ, LV = LY::LV, RTW = LY::RTW, NVT = LY::NVT, NST = LY::NST;
    constexpr int QF = DK / 32;       // query fragments per lane
    constexpr int NJ = W / 2 + 1;     // key fragments reaching query block W
    constexpr int NJC = CH / 32;      // key fragments per chunk
    constexpr bool kKeepV = NVT * NJC * 4 <= 32;
    const int lane = tid & 63, g = lane >> 4, li = lane & 15;
    __bf16* Kb = lds;
    __bf16* Vb = lds + 2 * LY::KSZ;
    __bf16* Sb = Vb + 2 * LY::VSZ;

    frag qf[2][QF];
    float lgb[2];
    // (the helpers take the thread index as an argument: inside the loop it
    // is an opaque per-chunk copy, see below)
    auto load_chunk = [&](int c0, int tid) { in.load(rq, rk, rv, ra, c0, W, tid); };
    auto write_st = [&](__bf16* st, int tid) {
        const int lane = tid & 63, g = lane >> 4, li = lane & 15;
#pragma unroll
        for (int i = 0; i < RTW; ++i)
#pragma unroll
            for (int c = 0; c < NVT; ++c) {
                __bf16* dst = &st[(16 * c + li) * LQ + 16 * (W * RTW + i) + 4 * g];
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[r] = M::cvt(S[i][c][r]);
            }
    };
    auto stage = [&](auto bconst, int c0, int tid) {
        constexpr int b = decltype(bconst)::value;
        const int lane = tid & 63;
        stage_rows_raw<bf16_t, DK, NTHR>(in.kr, tid, Kb + b * LY::KSZ, LQ);
        stage_rows_raw<bf16_t, DV, NTHR>(in.vr, tid, Vb + b * LY::VSZ, LV);
#pragma unroll
        for (int kk = 0; kk < QF; ++kk) qf[b][kk] = __builtin_bit_cast(frag, in.qraw[kk]);
        lgb[b] = log2_prefix(__uint_as_float(in.araw), c0 + lane < t_end, lane);
    };

    stage(std::integral_constant<int, 0>{}, t_beg, tid);
    write_st(Sb, tid);
    load_chunk(t_beg + CH, tid);
    __syncthreads();

    auto iter = [&](auto bconst, int c0) {
        constexpr int b = decltype(bconst)::value;
        // Lane indices from an opaque copy every chunk: the per-lane LDS
        // addresses built from them are then computed next to their uses
        // instead of being hoisted out of the loop and held throughout.
        int tid_v = threadIdx.x;
        asm volatile("" : "+v"(tid_v));
        const int tid = tid_v, lane = tid & 63, g = lane >> 4, li = lane & 15;
        const __bf16* Kc = Kb + b * LY::KSZ;
        const __bf16* Vc = Vb + b * LY::VSZ;
        const __bf16* Sc = Sb + (NST == 2 ? b : 0) * LY::SSZ;
        const float lg = lgb[b];
        const float lq = __shfl(lg, 16 * W + li);    // this lane's query
        const float lend = __shfl(lg, CH - 1);

        // P^T tiles: keys 16kb.. x this wave's queries, decay-weighted
        v4f Pt[W + 1];
#pragma unroll
        for (int kb = 0; kb <= W; ++kb) {
            Pt[kb] = zero4();
#pragma unroll
            for (int kk = 0; kk < QF; ++kk) M::mma(Pt[kb], M::load16(&Kc[(16 * kb + li) * LQ + 32 * kk], g), qf[b][kk]);
#pragma unroll
            for (int r = 0; r < 4; ++r) Pt[kb][r] *= exp2_hw(lq - __shfl(lg, 16 * kb + 4 * g + r));
        }
        // keys after the query: the ratio may have overflowed; the select drops it
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (4 * g + r > li) Pt[W][r] = 0.f;
        frag pf[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) pf[j] = M::from_tiles(Pt[2 * j], (2 * j + 1 <= W) ? Pt[(2 * j + 1) <= W ? 2 * j + 1 : W] : zero4());

        frag vf[kKeepV ? NVT : 1][NJC];
        if constexpr (kKeepV) {
#pragma unroll
            for (int c = 0; c < NVT; ++c)
#pragma unroll
                for (int j = 0; j < NJC; ++j) vf[c][j] = M::load_tr(Vc, LV, 32 * j, 16 * c, lane);
        }
        auto vfrag = [&](int c, int j) -> frag {
            if constexpr (kKeepV) return vf[c][j];
            else return M::load_tr(Vc, LV, 32 * j, 16 * c, lane);
        };

        // output tiles: the state read scaled by gamma_query, plus V^T P^T
        const float gq = exp2_hw(lq);
        const int orow = c0 + 16 * W + li;
        auto out_tile = [&](int c) {
            v4f N = zero4();
#pragma unroll
            for (int kk = 0; kk < QF; ++kk) M::mma(N, M::load16(&Sc[(16 * c + li) * LQ + 32 * kk], g), qf[b][kk]);
            N *= gq;
#pragma unroll
            for (int j = 0; j < NJ; ++j) M::mma(N, vfrag(c, j), pf[j]);
            return N;
        };
        // Tiles c, c+1: one row-pair swap gives every lane 8 consecutive
        // columns (even groups 16c + 8(g/2).., odd groups 16(c+1) + 8(g/2)..)
#pragma unroll
        for (int c = 0; c < NVT; c += 2) {
            const v4f n0 = out_tile(c), n1 = out_tile(c + 1);
            const uint32_t a0 = pack_bf16x2(n0[0], n0[1]), a1 = pack_bf16x2(n0[2], n0[3]);
            const uint32_t b0 = pack_bf16x2(n1[0], n1[1]), b1 = pack_bf16x2(n1[2], n1[3]);
            const auto s0 = __builtin_amdgcn_permlane16_swap(a0, b0, false, false);
            const auto s1 = __builtin_amdgcn_permlane16_swap(a1, b1, false, false);
            const v4u x = v4u{(uint32_t)s0[0], (uint32_t)s1[0], (uint32_t)s0[1], (uint32_t)s1[1]};
            const int col = 16 * c + 16 * (g & 1) + 8 * (g >> 1);
            buf_store16_stream(ro, (uint32_t)((orow * DV + col) * 2), x);
        }

        // state update (this wave's dk rows): decay, then the keys scaled by
        // gamma_C / gamma_key in registers (slot s of group g <-> key
        // 32j + 4g + s, or 32j + 16 + 4g + s - 4)
        const float gC = exp2_hw(lend);
#pragma unroll
        for (int i = 0; i < RTW; ++i)
#pragma unroll
            for (int c = 0; c < NVT; ++c) S[i][c] *= gC;
#pragma unroll
        for (int j = 0; j < NJC; ++j) {
            float kf[8];
#pragma unroll
            for (int s = 0; s < 8; ++s)
                kf[s] = exp2_hw(lend - __shfl(lg, 32 * j + (s < 4 ? 4 * g + s : 16 + 4 * g + s - 4)));
#pragma unroll
            for (int i = 0; i < RTW; ++i) {
                frag a = M::load_tr(Kc, LQ, 32 * j, 16 * (W * RTW + i), lane);
#pragma unroll
                for (int s = 0; s < 8; ++s) a[s] = M::cvt((float)a[s] * kf[s]);
#pragma unroll
                for (int c = 0; c < NVT; ++c) M::mma(S[i][c], a, vfrag(c, j));
            }
        }

        // next chunk: stage it, start the one after (reads past the segment
        // end return zero, gates there count as 1)
        stage(std::integral_constant<int, b ^ 1>{}, c0 + CH, tid);
        load_chunk(c0 + 2 * CH, tid);
        if constexpr (NST == 1) __syncthreads();  // all reads of S^T done
        write_st(Sb + (NST == 2 ? (b ^ 1) : 0) * LY::SSZ, tid);
        __syncthreads();
    };
    // Pairs of chunks with no exit between them; a chunk past t_end reads
    // zeros, leaves the state unchanged and has its stores dropped.
    for (int c0 = t_beg; c0 < t_end; c0 += 2 * CH) {
        iter(std::integral_constant<int, 0>{}, c0);
        iter(std::integral_constant<int, 1>{}, c0 + CH);
    }
}

template <int DK, int DV, bool PACKED>
__global__ __launch_bounds__(NTHR) void ssd_output_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                          const bf16_t* __restrict__ v,
                                                          const float* __restrict__ alpha, bf16_t* __restrict__ o,
                                                          const float* __restrict__ state_in, float* S_out,
                                                          SegMap sm) {
    using LY = SL<DK, DV>;
    constexpr int RTW = LY::RTW, NVT = LY::NVT;
    __shared__ __align__(16) __bf16 lds[LY::LDS_BYTES / 2];
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, li = lane & 15;
    const int w = wave_id(tid);
    int h, nseq, seg;
    if constexpr (!PACKED) {  // (sequence, head)-major, segments consecutive
        const int vh = blockIdx.x / sm.G;
        seg = blockIdx.x % sm.G;
        nseq = vh / sm.H;
        h = vh % sm.H;
    } else {
        const int vs = blockIdx.x % sm.NS;
        h = blockIdx.x / sm.NS;
        nseq = sm.seq_of<true>(vs);
        seg = vs - sm.seg_base<true>(nseq);
    }
    const long slot = sm.slot<PACKED>(nseq, h) + seg;
    const long row0 = h * sm.hs + sm.start<PACKED>(nseq);
    const int t_beg = seg * sm.L, t_end = min(t_beg + sm.L, sm.length<PACKED>(nseq));
    const rsrc_t rq = make_rsrc(q + row0 * DK, (uint32_t)t_end * DK * 2);
    const rsrc_t rk = make_rsrc(k + row0 * DK, (uint32_t)t_end * DK * 2);
    const rsrc_t rv = make_rsrc(v + row0 * DV, (uint32_t)t_end * DV * 2);
    const rsrc_t ra = make_rsrc(alpha + row0, (uint32_t)t_end * 4);
    const rsrc_t ro = make_rsrc(o + row0 * DV, (uint32_t)t_end * DV * 2);
    SsdChunk<DK, DV> first;
    first.load(rq, rk, rv, ra, t_beg, w, tid);

    v4f S[RTW][NVT];
    const float* sin = state_in + slot * DK * DV;
#pragma unroll
    for (int i = 0; i < RTW; ++i)
#pragma unroll
        for (int c = 0; c < NVT; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) S[i][c][r] = sin[(16 * (w * RTW + i) + 4 * g + r) * DV + 16 * c + li];

    switch (w) {
        case 0: ssd_output_pass<DK, DV, 0>(rq, rk, rv, ra, ro, t_beg, t_end, S, first, lds, tid); break;
        case 1: ssd_output_pass<DK, DV, 1>(rq, rk, rv, ra, ro, t_beg, t_end, S, first, lds, tid); break;
        case 2: ssd_output_pass<DK, DV, 2>(rq, rk, rv, ra, ro, t_beg, t_end, S, first, lds, tid); break;
        default: ssd_output_pass<DK, DV, 3>(rq, rk, rv, ra, ro, t_beg, t_end, S, first, lds, tid); break;
    }

    if (seg == sm.segs<PACKED>(nseq) - 1 && S_out) {
        float* dst = S_out + ((long)nseq * sm.H + h) * DK * DV;
#pragma unroll
        for (int i = 0; i < RTW; ++i)
#pragma unroll
            for (int c = 0; c < NVT; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(16 * (w * RTW + i) + 4 * g + r) * DV + 16 * c + li] = S[i][c][r];
    }
}

template <int DK, int DV, bool PACKED>
hipError_t launch_packing(const bf16_t* q, const bf16_t* k, const bf16_t* v, const float* alpha, const float* S0,
                        bf16_t* o, float* S_out, const SegMap& sm, float* ws, hipStream_t stream) {
    const size_t slots = (size_t)sm.H * sm.NS;
    constexpr int E = DK * DV;
    float* map_n = ws;
    float* state_in = map_n + slots * E;
    float* map_l = state_in + slots * E;
    hipError_t err;
    if (sm.NS > sm.N) {
        ssd_segment_kernel<DK, DV, PACKED><<<dim3(sm.H * (sm.NS - sm.N)), dim3(NTHR), 0, stream>>>(k, v, alpha, map_n, map_l,
                                                                                          sm);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    const long groups = (long)sm.N * sm.H * (E / 4);
    ssd_compose_kernel<E, PACKED><<<dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, stream>>>(map_n, map_l, S0,
                                                                                           state_in, sm);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    ssd_output_kernel<DK, DV, PACKED><<<dim3(sm.H * sm.NS), dim3(NTHR), 0, stream>>>(q, k, v, alpha, o, state_in, S_out, sm);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_typed(const bf16_t* q, const bf16_t* k, const bf16_t* v, const float* alpha, const float* S0,
                        bf16_t* o, float* S_out, const SegMap& sm, float* ws, hipStream_t stream) {
    return sm.packed() ? launch_packing<DK, DV, true>(q, k, v, alpha, S0, o, S_out, sm, ws, stream)
                       : launch_packing<DK, DV, false>(q, k, v, alpha, S0, o, S_out, sm, ws, stream);
}

}  // namespace

size_t ssd_ws_floats(long slots, int dk, int dv) {
    return (size_t)slots * (2 * (size_t)dk * dv + 1);
}

hipError_t launch_ssd_forward(const void* q, const void* k, const void* v, const float* alpha, const float* S0,
                              void* o, float* S_out, const SegMap& sm, int dk, int dv, int dtype,
                              float* ws, hipStream_t stream) {
    if (dtype != 1) return hipErrorInvalidValue;
    const bf16_t* qb = static_cast<const bf16_t*>(q);
    const bf16_t* kb = static_cast<const bf16_t*>(k);
    const bf16_t* vb = static_cast<const bf16_t*>(v);
    bf16_t* ob = static_cast<bf16_t*>(o);
#define SSD_CASE(A, B) \
    if (dk == A && dv == B) return launch_typed<A, B>(qb, kb, vb, alpha, S0, ob, S_out, sm, ws, stream);
    SSD_CASE(64, 64)
    SSD_CASE(64, 128)
    SSD_CASE(128, 64)
    SSD_CASE(128, 128)
#undef SSD_CASE
    return hipErrorInvalidValue;
}

}  // namespace la
