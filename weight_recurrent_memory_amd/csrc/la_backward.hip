// Backward pass of causal ELU+1 linear attention on gfx950 (bf16 inputs,
// fp32 accumulation and states).
//
// "AIGC 基本功｜线性、循环与记忆架构-LinearMem" §03 notes that storing every
// step's state makes training memory grow with the length, and that prefix
// sums, chunking and recomputation in the backward pass remove that cost;
// §06 asks for training and decoding to be validated separately.  Nothing
// of the forward pass is stored here: the chunk states are recomputed.
//
// For the loss L = sum_t dO_t . o_t + <dS_T, S_T> + <dz_T, z_T>, with
// num_t = phi(q_t)^T S_t, den_t = phi(q_t)^T z_t + eps, o_t = num_t / den_t:
//   dnum_t = dO_t / den_t,  dden_t = -(dO_t . num_t) / den_t^2,
//   dphi(q_t) = S_t dnum_t + z_t dden_t,
//   G(t) = [dS_T | dz_T] + sum_{s >= t} phi(q_s) [dnum_s | dden_s]^T,
//   dphi(k_t) = G_S(t) v_t + G_z(t),  dv_t = G_S(t)^T phi(k_t),
//   dS_0 = G_S(0), dz_0 = G_z(0),  d u = dphi(u) phi'(u).
// Over a chunk entered with state S' = [S | z] and left with gradient state
// G' = [G_S | G_z] (the later chunks' sum), with P = tril(phi(Q) phi(K)^T)
// and M = tril(dN' V'^T) (dN' = [dN | dden], V' = [V | 1]):
//   dphi(Q) = M phi(K) + dN' S'^T,   dphi(K) = M^T phi(Q) + V' G'^T,
//   dV = P^T dN + phi(K) G_S,        G' += phi(Q)^T dN'.
// phi'(u) is 1 for u > 0 and e^u = phi(u) otherwise, i.e. min(phi(u), 1).
//
// Five launches, sequence-parallel over segments like the forward pass:
//   lab_segsum   A_g = sum over segment g of phi(K)^T [V | 1] (all segments but the last)
//   lab_prefix   S_in(g+1) = S_in(g) + A_g, elementwise
//   lab_fwd      chunk loop from S_in(g): dq, the per-token 1/den and dden,
//                and Gseg(g) = sum over the segment of phi(Q)^T dN'
//   lab_suffix   G_in(g) = [dS_T | dz_T] + sum_{g' > g} Gseg(g'); dS_0, dz_0
//   lab_bwd      chunk loop backward from G_in(g): dk, dv
// Each chunk loop holds its running state in MFMA accumulators (wave w owns
// dk rows 16 w dk/64 ..) and shares it with the other waves through a bf16
// transposed copy in LDS, as the forward pass does.
#include "common.hpp"
#include "kernels.hpp"

namespace la {

namespace {

constexpr int CH = kChunk;
constexpr int NT = 256;  // four waves

typedef unsigned v2u __attribute__((ext_vector_type(2)));

// Four bf16 (8 bytes) through a buffer resource: dropped past its end.
__device__ __forceinline__ void store4_bf16(rsrc_t r, uint32_t off, const float (&x)[4]) {
    const v2u pk = v2u{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    __builtin_amdgcn_raw_buffer_store_b64(pk, r, off, 0, 0);
}

template <int DK, int DV>
struct BL {
    static constexpr int LQ = DK + 8;          // bf16 rows with k = dk: phi(Q), phi(K), S'^T, G'^T
    static constexpr int LV = DV + 8;          // bf16 rows of V and of dN
    static constexpr int RTW = DK / 64;        // dk row tiles of the running state per wave
    static constexpr int NVT = DV / 16;        // value column tiles
    static constexpr int NCT = NVT + 1;        // + the z (or G_z) tile, 16 equal columns
    static constexpr int E = DK * DV + DK;     // floats of one [S | z] state
    static constexpr int CQ = CH * LQ, CV = CH * LV, ST = (DV + 16) * LQ;
};

// LDS element offsets of the chunk buffers (single-buffered: staged at the
// top of each chunk from registers that were loaded one chunk earlier).
template <int DK, int DV>
struct BLds {
    using Y = BL<DK, DV>;
    // N, NL: dN' as hi and lo bf16 parts (the reverse sweep's M tiles use both).
    // S, SL: the transposed state copy, hi and lo parts; the lo part (used by
    // the forward sweep's dq) only where the LDS has room for it.
    static constexpr int K = 0, V = K + Y::CQ, Q = V + Y::CV, N = Q + Y::CQ, NL = N + Y::CV, S = NL + Y::CV;
    static constexpr bool STATE_LO = 2 * (S + 2 * Y::ST) + CH * 4 <= 160 * 1024;
    static constexpr int SL = S + Y::ST;
    static constexpr int BF16 = S + (STATE_LO ? 2 : 1) * Y::ST;  // bf16 elements
    static constexpr int BYTES = 2 * BF16 + CH * 4;  // + dden (fp32, one per query)
    // LDS reserved per workgroup: at least 56 KB.  At d = 64 the sweeps need
    // 48.6 KB; reserving 56 KB measured 122-126 us per call against
    // 127.5-133 us (same code and registers, two workgroups per CU either way
    // by registers), so only the placement of workgroups on CUs differs.
    static constexpr int RESERVED = BYTES > 56 * 1024 ? BYTES : 56 * 1024;
};

// The transposed bf16 copy of a running state tile set X[RTW][NCT] (rows dk
// 16 (w RTW + i) + 4g + r, columns 16c + li) into st: row = column of X.
// With lo non-null, also the rounding remainder: lo = bf16(x - hi).
template <int DK, int DV>
__device__ __forceinline__ void write_state_t(const v4f (&X)[BL<DK, DV>::RTW][BL<DK, DV>::NCT], __bf16* st, int w,
                                              int lane, __bf16* lo = nullptr) {
    using Y = BL<DK, DV>;
    const int g = lane >> 4, li = lane & 15;
#pragma unroll
    for (int i = 0; i < Y::RTW; ++i)
#pragma unroll
        for (int c = 0; c < Y::NCT; ++c) {
            const int off = (16 * c + li) * Y::LQ + 16 * (w * Y::RTW + i) + 4 * g;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const __bf16 hi = Mma<bf16_t>::cvt(X[i][c][r]);
                st[off + r] = hi;
                if (lo) lo[off + r] = Mma<bf16_t>::cvt(X[i][c][r] - (float)hi);
            }
        }
}

// Row-major [dk][dv] + z of a state <-> tiles X[RTW][NCT] (z in all 16 columns of the last tile).
template <int DK, int DV>
__device__ __forceinline__ void load_state(const float* src, v4f (&X)[BL<DK, DV>::RTW][BL<DK, DV>::NCT], int w,
                                           int lane) {
    using Y = BL<DK, DV>;
    const int g = lane >> 4, li = lane & 15;
#pragma unroll
    for (int i = 0; i < Y::RTW; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * (w * Y::RTW + i) + 4 * g + r;
#pragma unroll
            for (int c = 0; c < Y::NVT; ++c) X[i][c][r] = src[row * DV + 16 * c + li];
            X[i][Y::NCT - 1][r] = src[DK * DV + row];
        }
}

template <int DK, int DV>
__device__ __forceinline__ void store_state(float* dst, const v4f (&X)[BL<DK, DV>::RTW][BL<DK, DV>::NCT], int w,
                                            int lane) {
    using Y = BL<DK, DV>;
    const int g = lane >> 4, li = lane & 15;
#pragma unroll
    for (int i = 0; i < Y::RTW; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * (w * Y::RTW + i) + 4 * g + r;
#pragma unroll
            for (int c = 0; c < Y::NVT; ++c) dst[row * DV + 16 * c + li] = X[i][c][r];
            if (li == 0) dst[DK * DV + row] = X[i][Y::NCT - 1][r];
        }
}

// ------------------------------------------------------------- lab_segsum
template <int DK, int DV>
__global__ __launch_bounds__(NT) void lab_segsum_kernel(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                                                        float* __restrict__ agg, int T, int L, int G) {
    using Y = BL<DK, DV>;
    using M = Mma<bf16_t>;
    typedef M::frag frag;
    constexpr int RTW = Y::RTW, NCT = Y::NCT, NVT = Y::NVT;
    __shared__ __align__(16) __bf16 lds[Y::CQ + Y::CV];
    __bf16* Ks = lds;
    __bf16* Vs = lds + Y::CQ;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = wave_id(tid);
    const int head = blockIdx.x / (G - 1), seg = blockIdx.x % (G - 1);
    const int t0 = seg * L, t1 = min(t0 + L, T);
    const rsrc_t rk = make_rsrc(k + (long)head * T * DK, (uint32_t)t1 * DK * 2);
    const rsrc_t rv = make_rsrc(v + (long)head * T * DV, (uint32_t)t1 * DV * 2);
    ChunkRegs<bf16_t, DK, NT> kr;
    ChunkRegs<bf16_t, DV, NT> vr;
    kr.load_buf(rk, t0, tid);
    vr.load_buf(rv, t0, tid);
    v4f A[RTW][NCT];
#pragma unroll
    for (int i = 0; i < RTW; ++i)
#pragma unroll
        for (int c = 0; c < NCT; ++c) A[i][c] = zero4();
    for (int c0 = t0; c0 < t1; c0 += CH) {
        stage_rows_phi<bf16_t, DK, NT>(kr, t1 - c0, tid, Ks, Y::LQ);
        stage_rows_raw<bf16_t, DV, NT>(vr, tid, Vs, Y::LV);
        if (c0 + CH < t1) {
            kr.load_buf(rk, c0 + CH, tid);
            vr.load_buf(rv, c0 + CH, tid);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < CH / 32; ++j)
#pragma unroll
            for (int i = 0; i < RTW; ++i) {
                const frag a = M::load_tr(Ks, Y::LQ, 32 * j, 16 * (w * RTW + i), lane);
#pragma unroll
                for (int c = 0; c < NCT; ++c)
                    M::mma(A[i][c], a, c < NVT ? M::load_tr(Vs, Y::LV, 32 * j, 16 * c, lane) : M::ones());
            }
        __syncthreads();
    }
    store_state<DK, DV>(agg + ((long)head * G + seg) * Y::E, A, w, lane);
}

// ------------------------------------------------------------- lab_prefix / lab_suffix
// S_in(0) = [S0 | z0] (or 0), S_in(g+1) = S_in(g) + A_g.  Thread i owns
// element i of one head's state; the segments are taken in batches whose
// loads are all issued before the first add (one memory latency per batch).
constexpr int kScanBatch = 8;

template <int DK, int DV>
__global__ __launch_bounds__(256) void lab_prefix_kernel(const float* __restrict__ agg, const float* S0,
                                                         const float* z0, float* __restrict__ state_in, int HT,
                                                         int G) {
    constexpr int E = BL<DK, DV>::E;
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long)HT * E) return;
    const int head = (int)(idx / E), e = (int)(idx % E);
    const float* ah = agg + (long)head * G * E + e;
    float* sh = state_in + (long)head * G * E + e;
    float s = e < DK * DV ? (S0 ? S0[(long)head * DK * DV + e] : 0.f) : (z0 ? z0[(long)head * DK + e - DK * DV] : 0.f);
    sh[0] = s;
    for (int g0 = 0; g0 + 1 < G; g0 += kScanBatch) {
        float a[kScanBatch];
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u)
            if (g0 + u + 1 < G) a[u] = ah[(long)(g0 + u) * E];
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u)
            if (g0 + u + 1 < G) {
                s += a[u];
                sh[(long)(g0 + u + 1) * E] = s;
            }
    }
}

// G_in(G-1) = [dS_T | dz_T] (or 0), G_in(g) = G_in(g+1) + Gseg(g+1); then
// [dS_0 | dz_0] = G_in(0) + Gseg(0).  Batched like the prefix.
template <int DK, int DV>
__global__ __launch_bounds__(256) void lab_suffix_kernel(const float* __restrict__ gseg, const float* dS_T,
                                                         const float* dz_T, float* __restrict__ grad_in,
                                                         float* dS0, float* dz0, int HT, int G) {
    constexpr int E = BL<DK, DV>::E;
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long)HT * E) return;
    const int head = (int)(idx / E), e = (int)(idx % E);
    const bool sz = e < DK * DV;
    const float* gh = gseg + (long)head * G * E + e;
    float* oh = grad_in + (long)head * G * E + e;
    float s = sz ? (dS_T ? dS_T[(long)head * DK * DV + e] : 0.f) : (dz_T ? dz_T[(long)head * DK + e - DK * DV] : 0.f);
    for (int g0 = G - 1; g0 >= 0; g0 -= kScanBatch) {
        float a[kScanBatch];
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u)
            if (g0 - u >= 0) a[u] = gh[(long)(g0 - u) * E];
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u)
            if (g0 - u >= 0) {
                oh[(long)(g0 - u) * E] = s;
                s += a[u];
            }
    }
    if (sz) {
        if (dS0) dS0[(long)head * DK * DV + e] = s;
    } else if (dz0) {
        dz0[(long)head * DK + e - DK * DV] = s;
    }
}

// A B-operand fragment whose 16 columns all equal x[k] (k = the contraction
// index of the standard slot order over keys or queries 32kb..32kb+31).
__device__ __forceinline__ Mma<bf16_t>::frag broadcast_frag(const float* x, int kb, int g) {
    Mma<bf16_t>::frag f;
#pragma unroll
    for (int s = 0; s < 8; ++s) f[s] = Mma<bf16_t>::cvt(x[32 * kb + (s < 4 ? 4 * g + s : 16 + 4 * g + s - 4)]);
    return f;
}

// ------------------------------------------------------------- lab_fwd
// Wave W owns the chunk's queries 16W..16W+15 (their dq) and dk rows
// 16 W RTW .. of the running state S' and of Gseg.
template <int DK, int DV, int W>
__device__ __forceinline__ void lab_fwd_pass(rsrc_t rq, rsrc_t rk, rsrc_t rv, rsrc_t rdo, rsrc_t rtok, rsrc_t rdq,
                                             int t_beg, int t_end, float eps,
                                             v4f (&S)[BL<DK, DV>::RTW][BL<DK, DV>::NCT],
                                             v4f (&Gs)[BL<DK, DV>::RTW][BL<DK, DV>::NCT], __bf16* lds, int tid) {
    using Y = BL<DK, DV>;
    using LO = BLds<DK, DV>;
    using M = Mma<bf16_t>;
    typedef M::frag frag;
    constexpr int LQ = Y::LQ, LV = Y::LV, RTW = Y::RTW, NVT = Y::NVT, NCT = Y::NCT;
    constexpr int QF = DK / 32, NJ = W / 2 + 1, NJC = CH / 32;
    __bf16* Ks = lds + LO::K;
    __bf16* Vs = lds + LO::V;
    __bf16* Qs = lds + LO::Q;
    __bf16* Ns = lds + LO::N;
    __bf16* Sts = lds + LO::S;
    __bf16* Stl = LO::STATE_LO ? lds + LO::SL : nullptr;
    float* Dd = reinterpret_cast<float*>(lds + LO::BF16);

    ChunkRegs<bf16_t, DK, NT> kr, qr;
    ChunkRegs<bf16_t, DV, NT> vr;
    uint2 dor[NVT];  // this lane's dO: query 16W + li, columns 16c + 4g .. +3
    auto load_chunk = [&](int c0) {
        const int lane = tid & 63, g = lane >> 4, li = lane & 15;
        kr.load_buf(rk, c0, tid);
        qr.load_buf(rq, c0, tid);
        vr.load_buf(rv, c0, tid);
#pragma unroll
        for (int c = 0; c < NVT; ++c) {
            const uint32_t off = (uint32_t)(((c0 + 16 * W + li) * DV + 16 * c + 4 * g) * 2);
            dor[c].x = __builtin_amdgcn_raw_buffer_load_b32(rdo, off, 0, 0);
            dor[c].y = __builtin_amdgcn_raw_buffer_load_b32(rdo, off + 4, 0, 0);
        }
    };
    load_chunk(t_beg);

    for (int c0 = t_beg; c0 < t_end; c0 += CH) {
        // Lane indices from an opaque copy every chunk, so the per-lane LDS
        // addresses are computed next to their uses, not held across the loop.
        int tid_v = tid;
        asm volatile("" : "+v"(tid_v));
        const int lane = tid_v & 63, g = lane >> 4, li = lane & 15;
        // ---- stage the chunk and the state entering it; start the next chunk
        stage_rows_phi<bf16_t, DK, NT>(kr, t_end - c0, tid_v, Ks, LQ);
        stage_rows_phi<bf16_t, DK, NT>(qr, t_end - c0, tid_v, Qs, LQ);
        stage_rows_raw<bf16_t, DV, NT>(vr, tid_v, Vs, LV);
        write_state_t<DK, DV>(S, Sts, W, lane, Stl);
        v4f dOt[NVT];
#pragma unroll
        for (int c = 0; c < NVT; ++c) {
            const uint32_t wlo = dor[c].x, whi = dor[c].y;
            dOt[c] = v4f{__uint_as_float(wlo << 16), __uint_as_float(wlo & 0xffff0000u), __uint_as_float(whi << 16),
                         __uint_as_float(whi & 0xffff0000u)};
        }
        if (c0 + CH < t_end) load_chunk(c0 + CH);
        __syncthreads();

        // ---- P^T tiles (keys 16kb.. x this wave's queries), numerator and denominator
        frag qf[QF];
#pragma unroll
        for (int kk = 0; kk < QF; ++kk) qf[kk] = M::load16(&Qs[(16 * W + li) * LQ + 32 * kk], g);
        v4f Pt[W + 1];
#pragma unroll
        for (int kb = 0; kb <= W; ++kb) {
            Pt[kb] = zero4();
#pragma unroll
            for (int kk = 0; kk < QF; ++kk) M::mma(Pt[kb], M::load16(&Ks[(16 * kb + li) * LQ + 32 * kk], g), qf[kk]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (4 * g + r > li) Pt[W][r] = 0.f;
        frag pf[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) pf[j] = M::from_tiles(Pt[2 * j], (2 * j + 1 <= W) ? Pt[(2 * j + 1) <= W ? 2 * j + 1 : W] : zero4());
        v4f D = zero4();
#pragma unroll
        for (int j = 0; j < NJ; ++j) M::mma(D, M::ones(), pf[j]);
#pragma unroll
        for (int kk = 0; kk < QF; ++kk) M::mma(D, M::load16(&Sts[(DV + li) * LQ + 32 * kk], g), qf[kk]);
        const float inv = fast_rcp(D[0] + eps);
        v4f dNt[NVT];
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < NVT; ++c) {
            v4f N = zero4();
#pragma unroll
            for (int j = 0; j < NJ; ++j) M::mma(N, M::load_tr(Vs, LV, 32 * j, 16 * c, lane), pf[j]);
#pragma unroll
            for (int kk = 0; kk < QF; ++kk) M::mma(N, M::load16(&Sts[(16 * c + li) * LQ + 32 * kk], g), qf[kk]);
#pragma unroll
            for (int r = 0; r < 4; ++r) dot += dOt[c][r] * N[r];
            dNt[c] = dOt[c] * inv;
        }
        dot += __shfl_xor(dot, 16);
        dot += __shfl_xor(dot, 32);
        const float dden = -dot * inv * inv;
        // per-token scalars for the backward sweep; dN' rows for the other waves
        if (g == 0) {
            const uint32_t off = (uint32_t)((c0 + 16 * W + li) * 8);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(inv), rtok, off, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dden), rtok, off + 4, 0, 0);
            Dd[16 * W + li] = dden;
        }
#pragma unroll
        for (int c = 0; c < NVT; ++c) {
            uint2 pk;
            pk.x = pack_bf16x2(dNt[c][0], dNt[c][1]);
            pk.y = pack_bf16x2(dNt[c][2], dNt[c][3]);
            *reinterpret_cast<uint2*>(&Ns[(16 * W + li) * LV + 16 * c + 4 * g]) = pk;
        }

        // ---- M^T tiles (keys 16kb.. x this wave's queries): V dN^T + dden, causal.
        // M[t][i] = dN_t . (v_i - o_t) cancels where v_i is near o_t (the
        // first tokens above all): dN enters as hi + lo bf16 parts, so its
        // rounding does not set the error of the difference.
        frag dnh[NVT / 2], dnl[NVT / 2];
#pragma unroll
        for (int cc = 0; cc < NVT / 2; ++cc) M::split_tiles(dNt[2 * cc], dNt[2 * cc + 1], dnh[cc], dnl[cc]);
        v4f Mt[W + 1];
#pragma unroll
        for (int kb = 0; kb <= W; ++kb) {
            Mt[kb] = zero4();
#pragma unroll
            for (int cc = 0; cc < NVT / 2; ++cc) {
                const frag va = M::load(&Vs[(16 * kb + li) * LV + 32 * cc], g);
                M::mma(Mt[kb], va, dnh[cc]);
                M::mma(Mt[kb], va, dnl[cc]);
            }
            Mt[kb] += dden;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (4 * g + r > li) Mt[W][r] = 0.f;

        // ---- dphi(Q)^T tiles (dk rows x this wave's queries) -> dq
#pragma unroll
        for (int t = 0; t < DK / 16; ++t) {
            v4f acc = zero4();
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                M::mma(acc, M::load_tr(Ks, LQ, 32 * j, 16 * t, lane),
                       M::from_tiles(Mt[2 * j], (2 * j + 1 <= W) ? Mt[(2 * j + 1) <= W ? 2 * j + 1 : W] : zero4()));
            // S dN + z dden nearly cancel where o is near the history's mean
            // value: state and dN both enter as hi + lo parts (where the
            // state's lo part fits in LDS)
#pragma unroll
            for (int cc = 0; cc < NVT / 2; ++cc) {
                const frag sa = M::load_tr(Sts, LQ, 32 * cc, 16 * t, lane);
                M::mma(acc, sa, dnh[cc]);
                M::mma(acc, sa, dnl[cc]);
                if constexpr (LO::STATE_LO) M::mma(acc, M::load_tr(Stl, LQ, 32 * cc, 16 * t, lane), dnh[cc]);
            }
            const v4bf zr = *reinterpret_cast<const v4bf*>(&Sts[DV * LQ + 16 * t + 4 * g]);
            v4f zf = v4f{(float)zr[0], (float)zr[1], (float)zr[2], (float)zr[3]};
            if constexpr (LO::STATE_LO) {
                const v4bf zl = *reinterpret_cast<const v4bf*>(&Stl[DV * LQ + 16 * t + 4 * g]);
#pragma unroll
                for (int r = 0; r < 4; ++r) zf[r] += (float)zl[r];
            }
            const v4bf fq = *reinterpret_cast<const v4bf*>(&Qs[(16 * W + li) * LQ + 16 * t + 4 * g]);
            float o4[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) o4[r] = (acc[r] + zf[r] * dden) * fminf((float)fq[r], 1.f);
            store4_bf16(rdq, (uint32_t)(((c0 + 16 * W + li) * DK + 16 * t + 4 * g) * 2), o4);
        }
        __syncthreads();  // dN' of every wave in LDS

        // ---- Gseg += phi(Q)^T dN' and S' += phi(K)^T [V | 1] (this wave's dk rows)
#pragma unroll
        for (int qq = 0; qq < NJC; ++qq)
#pragma unroll
            for (int i = 0; i < RTW; ++i) {
                const frag aq = M::load_tr(Qs, LQ, 32 * qq, 16 * (W * RTW + i), lane);
                const frag ak = M::load_tr(Ks, LQ, 32 * qq, 16 * (W * RTW + i), lane);
#pragma unroll
                for (int c = 0; c < NCT; ++c) {
                    M::mma(Gs[i][c], aq, c < NVT ? M::load_tr(Ns, LV, 32 * qq, 16 * c, lane) : broadcast_frag(Dd, qq, g));
                    M::mma(S[i][c], ak, c < NVT ? M::load_tr(Vs, LV, 32 * qq, 16 * c, lane) : M::ones());
                }
            }
        __syncthreads();  // before the next chunk overwrites the buffers
    }
}

template <int DK, int DV>
__global__ __launch_bounds__(NT) void lab_fwd_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                     const bf16_t* __restrict__ v, const bf16_t* __restrict__ dO,
                                                     const float* __restrict__ state_in, float* __restrict__ tok,
                                                     float* __restrict__ gseg, bf16_t* __restrict__ dq, int T, int L,
                                                     int G, float eps) {
    using Y = BL<DK, DV>;
    using LO = BLds<DK, DV>;
    constexpr int RTW = Y::RTW, NCT = Y::NCT;
    __shared__ __align__(16) __bf16 lds[LO::RESERVED / 2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = wave_id(tid);
    const int head = blockIdx.x / G, seg = blockIdx.x % G;
    const int t_beg = seg * L, t_end = min(t_beg + L, T);
    const rsrc_t rq = make_rsrc(q + (long)head * T * DK, (uint32_t)t_end * DK * 2);
    const rsrc_t rk = make_rsrc(k + (long)head * T * DK, (uint32_t)t_end * DK * 2);
    const rsrc_t rv = make_rsrc(v + (long)head * T * DV, (uint32_t)t_end * DV * 2);
    const rsrc_t rdo = make_rsrc(dO + (long)head * T * DV, (uint32_t)t_end * DV * 2);
    const rsrc_t rtok = make_rsrc(tok + (long)head * T * 2, (uint32_t)t_end * 8);
    const rsrc_t rdq = make_rsrc(dq + (long)head * T * DK, (uint32_t)t_end * DK * 2);
    v4f S[RTW][NCT], Gs[RTW][NCT];
    load_state<DK, DV>(state_in + ((long)head * G + seg) * Y::E, S, w, lane);
#pragma unroll
    for (int i = 0; i < RTW; ++i)
#pragma unroll
        for (int c = 0; c < NCT; ++c) Gs[i][c] = zero4();
    switch (w) {
        case 0: lab_fwd_pass<DK, DV, 0>(rq, rk, rv, rdo, rtok, rdq, t_beg, t_end, eps, S, Gs, lds, tid); break;
        case 1: lab_fwd_pass<DK, DV, 1>(rq, rk, rv, rdo, rtok, rdq, t_beg, t_end, eps, S, Gs, lds, tid); break;
        case 2: lab_fwd_pass<DK, DV, 2>(rq, rk, rv, rdo, rtok, rdq, t_beg, t_end, eps, S, Gs, lds, tid); break;
        default: lab_fwd_pass<DK, DV, 3>(rq, rk, rv, rdo, rtok, rdq, t_beg, t_end, eps, S, Gs, lds, tid); break;
    }
    store_state<DK, DV>(gseg + ((long)head * G + seg) * Y::E, Gs, w, lane);
}

// ------------------------------------------------------------- lab_bwd
// Chunks in reverse order from the segment end.  Wave W owns the chunk's
// keys 16W..16W+15 (their dk, dv) and dk rows 16 W RTW .. of G'.  The dN
// rows are rebuilt while staging from dO and the per-token 1/den; dden
// comes from the same record.
template <int DK, int DV, int W>
__device__ __forceinline__ void lab_bwd_pass(rsrc_t rq, rsrc_t rk, rsrc_t rv, rsrc_t rdo, rsrc_t rtok, rsrc_t rdk,
                                             rsrc_t rdv, int t_beg, int t_end,
                                             v4f (&Gp)[BL<DK, DV>::RTW][BL<DK, DV>::NCT], __bf16* lds, int tid) {
    using Y = BL<DK, DV>;
    using LO = BLds<DK, DV>;
    using M = Mma<bf16_t>;
    typedef M::frag frag;
    constexpr int LQ = Y::LQ, LV = Y::LV, RTW = Y::RTW, NVT = Y::NVT, NCT = Y::NCT;
    constexpr int QF = DK / 32, NJC = CH / 32;
    __bf16* Ks = lds + LO::K;
    __bf16* Vs = lds + LO::V;
    __bf16* Qs = lds + LO::Q;
    __bf16* Ns = lds + LO::N;
    __bf16* Nl = lds + LO::NL;
    __bf16* Gts = lds + LO::S;
    float* Dd = reinterpret_cast<float*>(lds + LO::BF16);

    ChunkRegs<bf16_t, DK, NT> kr, qr;
    ChunkRegs<bf16_t, DV, NT> vr, dr;
    float tinv[ChunkRegs<bf16_t, DV, NT>::NV];
    float tdd = 0.f;
    auto load_chunk = [&](int c0) {
        kr.load_buf(rk, c0, tid);
        qr.load_buf(rq, c0, tid);
        vr.load_buf(rv, c0, tid);
        dr.load_buf(rdo, c0, tid);
#pragma unroll
        for (int j = 0; j < ChunkRegs<bf16_t, DV, NT>::NV; ++j) {
            const int row = ChunkRegs<bf16_t, DV, NT>::row_of(j, tid);
            tinv[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rtok, (uint32_t)((c0 + row) * 8), 0, 0));
        }
        if (tid < CH) tdd = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rtok, (uint32_t)((c0 + tid) * 8 + 4), 0, 0));
    };
    const int nch = (t_end - t_beg + CH - 1) / CH;
    int c0 = t_beg + (nch - 1) * CH;
    load_chunk(c0);

    for (int it = 0; it < nch; ++it, c0 -= CH) {
        int tid_v = tid;
        asm volatile("" : "+v"(tid_v));
        const int lane = tid_v & 63, g = lane >> 4, li = lane & 15;
        // ---- stage the chunk (dN rebuilt from dO and 1/den) and G'^T; start the previous chunk
        stage_rows_phi<bf16_t, DK, NT>(kr, t_end - c0, tid_v, Ks, LQ);
        stage_rows_phi<bf16_t, DK, NT>(qr, t_end - c0, tid_v, Qs, LQ);
        stage_rows_raw<bf16_t, DV, NT>(vr, tid_v, Vs, LV);
#pragma unroll
        for (int j = 0; j < ChunkRegs<bf16_t, DV, NT>::NV; ++j) {
            const int row = ChunkRegs<bf16_t, DV, NT>::row_of(j, tid_v);
            const int col = ChunkRegs<bf16_t, DV, NT>::col_of(j, tid_v);
            float dn[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) dn[e] = dr.get(j, e) * tinv[j];
            uint4 x, y;
            x.x = pack_bf16x2(dn[0], dn[1]);
            x.y = pack_bf16x2(dn[2], dn[3]);
            x.z = pack_bf16x2(dn[4], dn[5]);
            x.w = pack_bf16x2(dn[6], dn[7]);
            const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
            uint32_t ys[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ys[e] = pack_bf16x2(dn[2 * e] - __uint_as_float(xs[e] << 16),
                                    dn[2 * e + 1] - __uint_as_float(xs[e] & 0xffff0000u));
            y = make_uint4(ys[0], ys[1], ys[2], ys[3]);
            *reinterpret_cast<uint4*>(&Ns[row * LV + col]) = x;
            *reinterpret_cast<uint4*>(&Nl[row * LV + col]) = y;
        }
        if (tid_v < CH) Dd[tid_v] = tdd;
        write_state_t<DK, DV>(Gp, Gts, W, lane);
        if (it + 1 < nch) load_chunk(c0 - CH);
        __syncthreads();

        // ---- M tiles (queries 16qb.. x this wave's keys): dN V^T + dden, causal (query >= key);
        // dN as hi + lo parts, as in the forward sweep (M cancels where v is near o)
        v4f Mq[CH / 16], Pq[CH / 16];
#pragma unroll
        for (int qb = 0; qb < CH / 16; ++qb) {
            Mq[qb] = zero4();
            Pq[qb] = zero4();
            if (qb >= W) {
#pragma unroll
                for (int cc = 0; cc < NVT / 2; ++cc) {
                    const frag vb = M::load(&Vs[(16 * W + li) * LV + 32 * cc], g);
                    M::mma(Mq[qb], M::load(&Ns[(16 * qb + li) * LV + 32 * cc], g), vb);
                    M::mma(Mq[qb], M::load(&Nl[(16 * qb + li) * LV + 32 * cc], g), vb);
                }
                const v4f dd = *reinterpret_cast<const v4f*>(&Dd[16 * qb + 4 * g]);
                Mq[qb] += dd;
#pragma unroll
                for (int kk = 0; kk < QF; ++kk)
                    M::mma(Pq[qb], M::load16(&Qs[(16 * qb + li) * LQ + 32 * kk], g),
                           M::load16(&Ks[(16 * W + li) * LQ + 32 * kk], g));
                if (qb == W) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (4 * g + r < li) {
                            Mq[qb][r] = 0.f;
                            Pq[qb][r] = 0.f;
                        }
                }
            }
        }

        // ---- dphi(K)^T tiles (dk rows x this wave's keys) -> dk
#pragma unroll
        for (int t = 0; t < DK / 16; ++t) {
            v4f acc = zero4();
#pragma unroll
            for (int qq = W / 2; qq < NJC; ++qq)
                M::mma(acc, M::load_tr(Qs, LQ, 32 * qq, 16 * t, lane), M::from_tiles(Mq[2 * qq], Mq[2 * qq + 1]));
#pragma unroll
            for (int cc = 0; cc < NVT / 2; ++cc)
                M::mma(acc, M::load_tr(Gts, LQ, 32 * cc, 16 * t, lane), M::load(&Vs[(16 * W + li) * LV + 32 * cc], g));
            const v4bf gz = *reinterpret_cast<const v4bf*>(&Gts[DV * LQ + 16 * t + 4 * g]);
            const v4bf fk = *reinterpret_cast<const v4bf*>(&Ks[(16 * W + li) * LQ + 16 * t + 4 * g]);
            float o4[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) o4[r] = (acc[r] + (float)gz[r]) * fminf((float)fk[r], 1.f);
            store4_bf16(rdk, (uint32_t)(((c0 + 16 * W + li) * DK + 16 * t + 4 * g) * 2), o4);
        }

        // ---- dV^T tiles (value columns x this wave's keys) -> dv
#pragma unroll
        for (int c = 0; c < NVT; ++c) {
            v4f acc = zero4();
#pragma unroll
            for (int qq = W / 2; qq < NJC; ++qq)
                M::mma(acc, M::load_tr(Ns, LV, 32 * qq, 16 * c, lane), M::from_tiles(Pq[2 * qq], Pq[2 * qq + 1]));
#pragma unroll
            for (int kk = 0; kk < QF; ++kk)
                M::mma(acc, M::load(&Gts[(16 * c + li) * LQ + 32 * kk], g), M::load(&Ks[(16 * W + li) * LQ + 32 * kk], g));
            const float o4[4] = {acc[0], acc[1], acc[2], acc[3]};
            store4_bf16(rdv, (uint32_t)(((c0 + 16 * W + li) * DV + 16 * c + 4 * g) * 2), o4);
        }

        // ---- G' += phi(Q)^T dN' (this wave's dk rows)
#pragma unroll
        for (int qq = 0; qq < NJC; ++qq)
#pragma unroll
            for (int i = 0; i < RTW; ++i) {
                const frag aq = M::load_tr(Qs, LQ, 32 * qq, 16 * (W * RTW + i), lane);
#pragma unroll
                for (int c = 0; c < NCT; ++c)
                    M::mma(Gp[i][c], aq, c < NVT ? M::load_tr(Ns, LV, 32 * qq, 16 * c, lane) : broadcast_frag(Dd, qq, g));
            }
        __syncthreads();  // before the next (earlier) chunk overwrites the buffers
    }
}

template <int DK, int DV>
__global__ __launch_bounds__(NT) void lab_bwd_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                     const bf16_t* __restrict__ v, const bf16_t* __restrict__ dO,
                                                     const float* __restrict__ tok, const float* __restrict__ grad_in,
                                                     bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, int T, int L,
                                                     int G) {
    using Y = BL<DK, DV>;
    using LO = BLds<DK, DV>;
    constexpr int RTW = Y::RTW, NCT = Y::NCT;
    __shared__ __align__(16) __bf16 lds[LO::RESERVED / 2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = wave_id(tid);
    const int head = blockIdx.x / G, seg = blockIdx.x % G;
    const int t_beg = seg * L, t_end = min(t_beg + L, T);
    const rsrc_t rq = make_rsrc(q + (long)head * T * DK, (uint32_t)t_end * DK * 2);
    const rsrc_t rk = make_rsrc(k + (long)head * T * DK, (uint32_t)t_end * DK * 2);
    const rsrc_t rv = make_rsrc(v + (long)head * T * DV, (uint32_t)t_end * DV * 2);
    const rsrc_t rdo = make_rsrc(dO + (long)head * T * DV, (uint32_t)t_end * DV * 2);
    const rsrc_t rtok = make_rsrc(tok + (long)head * T * 2, (uint32_t)t_end * 8);
    const rsrc_t rdk = make_rsrc(dk + (long)head * T * DK, (uint32_t)t_end * DK * 2);
    const rsrc_t rdv = make_rsrc(dv + (long)head * T * DV, (uint32_t)t_end * DV * 2);
    v4f Gp[RTW][NCT];
    load_state<DK, DV>(grad_in + ((long)head * G + seg) * Y::E, Gp, w, lane);
    switch (w) {
        case 0: lab_bwd_pass<DK, DV, 0>(rq, rk, rv, rdo, rtok, rdk, rdv, t_beg, t_end, Gp, lds, tid); break;
        case 1: lab_bwd_pass<DK, DV, 1>(rq, rk, rv, rdo, rtok, rdk, rdv, t_beg, t_end, Gp, lds, tid); break;
        case 2: lab_bwd_pass<DK, DV, 2>(rq, rk, rv, rdo, rtok, rdk, rdv, t_beg, t_end, Gp, lds, tid); break;
        default: lab_bwd_pass<DK, DV, 3>(rq, rk, rv, rdo, rtok, rdk, rdv, t_beg, t_end, Gp, lds, tid); break;
    }
}

template <int DK, int DV>
hipError_t launch_typed(const bf16_t* q, const bf16_t* k, const bf16_t* v, const float* S0, const float* z0,
                        const bf16_t* dO, const float* dS_T, const float* dz_T, bf16_t* dq, bf16_t* dk, bf16_t* dv,
                        float* dS0, float* dz0, int HT, int T, float eps, const LaPlan& plan, float* ws,
                        hipStream_t stream) {
    using Y = BL<DK, DV>;
    const int G = plan.G, L = plan.L;
    const size_t slots = (size_t)HT * G;
    float* agg = ws;                           // A_g, then reused for Gseg(g)
    float* state_in = agg + slots * Y::E;      // S_in(g), then reused for G_in(g)
    float* tok = state_in + slots * Y::E;      // [HT][T][2]: 1/den, dden
    hipError_t err;
    if (G > 1) {
        lab_segsum_kernel<DK, DV><<<dim3(HT * (G - 1)), dim3(NT), 0, stream>>>(k, v, agg, T, L, G);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    const unsigned eblocks = (unsigned)(((long)HT * Y::E + 255) / 256);
    lab_prefix_kernel<DK, DV><<<dim3(eblocks), dim3(256), 0, stream>>>(agg, S0, z0, state_in, HT, G);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    lab_fwd_kernel<DK, DV><<<dim3(HT * G), dim3(NT), 0, stream>>>(q, k, v, dO, state_in, tok, agg, dq, T, L, G, eps);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    lab_suffix_kernel<DK, DV><<<dim3(eblocks), dim3(256), 0, stream>>>(agg, dS_T, dz_T, state_in, dS0, dz0, HT, G);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    lab_bwd_kernel<DK, DV><<<dim3(HT * G), dim3(NT), 0, stream>>>(q, k, v, dO, tok, state_in, dk, dv, T, L, G);
    return hipGetLastError();
}

}  // namespace

size_t la_backward_ws_floats(int HT, int T, int dk, int dv, const LaPlan& plan) {
    return (size_t)HT * plan.G * 2 * ((size_t)dk * dv + dk) + (size_t)HT * T * 2;
}

size_t la_backward_lds_bytes(int dk, int dv) {
#define LDS_CASE(A, B) \
    if (dk == A && dv == B) return BLds<A, B>::RESERVED;
    LDS_CASE(64, 64)
    LDS_CASE(64, 128)
    LDS_CASE(128, 64)
    LDS_CASE(128, 128)
#undef LDS_CASE
    return (size_t)1 << 30;
}

hipError_t launch_la_backward(const void* q, const void* k, const void* v, const float* S0, const float* z0,
                              const void* dO, const float* dS_T, const float* dz_T, void* dq, void* dk, void* dv,
                              float* dS0, float* dz0, int HT, int T, int dk_, int dv_, int dtype, float eps,
                              const LaPlan& plan, float* ws, hipStream_t stream) {
    if (dtype != 1) return hipErrorInvalidValue;
    const bf16_t* qb = static_cast<const bf16_t*>(q);
    const bf16_t* kb = static_cast<const bf16_t*>(k);
    const bf16_t* vb = static_cast<const bf16_t*>(v);
    const bf16_t* gb = static_cast<const bf16_t*>(dO);
#define BWD_CASE(A, B)                                                                                             \
    if (dk_ == A && dv_ == B)                                                                                      \
        return launch_typed<A, B>(qb, kb, vb, S0, z0, gb, dS_T, dz_T, static_cast<bf16_t*>(dq),                    \
                                  static_cast<bf16_t*>(dk), static_cast<bf16_t*>(dv), dS0, dz0, HT, T, eps, plan, ws, \
                                  stream);
    BWD_CASE(64, 64)
    BWD_CASE(64, 128)
    BWD_CASE(128, 64)
    BWD_CASE(128, 128)
#undef BWD_CASE
    return hipErrorInvalidValue;
}

}  // namespace la
