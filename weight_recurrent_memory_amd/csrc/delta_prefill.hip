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
// T is built in fp32: the four 16x16 diagonal blocks by forward substitution
// in registers, the off-diagonal blocks level by level,
//   T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj.
//
// Sequence parallelism.  Over a segment of chunks the rule is affine in the
// incoming state: S_out = M_g S_in + N_g.  Running the same chunk recurrence
// on a state started at 0 with the segment's values gives N_g; running it on a
// state started at I with zero values gives M_g (each state column evolves
// independently, so the two are separate workgroups).  Three launches:
//   delta_chunk<MAP>  (M_g, N_g) for every segment but the last
//   delta_compose     S_in(g+1) = M_g S_in(g) + N_g, fp32 MFMA, serial in g
//   delta_chunk<OUT>  the chunk loop from S_in(g), writing O (and S_T last)
#include "common.hpp"
#include "kernels.hpp"

namespace la {

namespace {

constexpr int CH = kChunk;
constexpr int NT = 512;  // eight waves
constexpr int NWV = 8;

template <int DK, int NS, bool OUT>
struct DL {
    static constexpr int LQ = DK + 8;  // bf16 rows with k = dk
    static constexpr int LV = NS + 8;  // bf16 rows of V
    static constexpr int LT = CH + 8;  // bf16 rows with k = token
    static constexpr int LF = CH + 4;  // fp32 rows of the C x C work matrix
    static constexpr int KS = CH * LQ * 2;          // K_c rows (read transposed too)
    static constexpr int WS = CH * LQ * 2;          // W rows
    static constexpr int QS = OUT ? CH * LQ * 2 : 0;
    static constexpr int XT = NS * LQ * 2;          // state^T (bf16)
    static constexpr int VS = CH * LV * 2;          // V_c rows (read transposed)
    static constexpr int UT = NS * LT * 2;          // (beta o U)^T
    static constexpr int TS = CH * LT * 2;          // T (bf16)
    static constexpr int AF = CH * LF * 4;          // A, then T blocks (fp32)
    static constexpr int BS = CH * 4;               // beta (fp32)
    static constexpr int TOTAL = KS + WS + QS + XT + VS + UT + TS + AF + BS;
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
    // state tiles (DK/16 x NS/16) over eight waves
    static constexpr int XR = DK / 16;
    static constexpr int XC = NS / 16;
    static constexpr int X_CPW = XR * XC / NWV;
    // C x NS tiles (4 x XC) over eight waves: row tile w%4, half the columns
    static constexpr int O_CPW = XC / 2;
    // W^T tiles (XR x 4) over eight waves
    static constexpr int W_TPW = 4 * XR / NWV;
};

// The ten lower 16x16 tiles of a 64x64 matrix: diagonal first.
__device__ __forceinline__ void lower_tile(int id, int& i, int& j) {
    if (id < 4) { i = id; j = id; }                // (0,0) (1,1) (2,2) (3,3)
    else if (id < 7) { i = id - 3; j = id - 4; }   // (1,0) (2,1) (3,2)
    else if (id < 9) { i = id - 5; j = id - 7; }   // (2,0) (3,1)
    else { i = 3; j = 0; }                         // (3,0)
}

template <int DK, int NS, bool OUT>
__global__ __launch_bounds__(NT) void delta_chunk_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ beta, bf16_t* __restrict__ o, const float* __restrict__ state_in,
    float* __restrict__ map_n, float* __restrict__ map_m, float* __restrict__ S_out, int T, int L,
    int G, int part_base) {
    using Y = DL<DK, NS, OUT>;
    using M = Mma<bf16_t>;
    using MF = Mma<float>;
    typedef M::frag frag;
    constexpr int LQ = Y::LQ, LT = Y::LT, LF = Y::LF;
    __shared__ __align__(16) unsigned char smem[Y::TOTAL];
    constexpr int LV = Y::LV;
    unsigned char* sp = smem;
    __bf16* Ks = reinterpret_cast<__bf16*>(sp);  sp += Y::KS;
    __bf16* Ws = reinterpret_cast<__bf16*>(sp);  sp += Y::WS;
    __bf16* Qs = reinterpret_cast<__bf16*>(sp);  sp += Y::QS;
    __bf16* Xt = reinterpret_cast<__bf16*>(sp);  sp += Y::XT;
    __bf16* Vs = reinterpret_cast<__bf16*>(sp);  sp += Y::VS;
    __bf16* Ut = reinterpret_cast<__bf16*>(sp);  sp += Y::UT;
    __bf16* Ts = reinterpret_cast<__bf16*>(sp);  sp += Y::TS;
    float* Af = reinterpret_cast<float*>(sp);
    float* Bs = Af + CH * LF;

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, li = lane & 15;
    const int w = wave_id(tid);
    int head, seg, part;
    if constexpr (OUT) {
        head = blockIdx.x / G;
        seg = blockIdx.x % G;
        part = 0;
    } else {
        head = blockIdx.x / (G - 1);
        seg = blockIdx.x % (G - 1);
        part = part_base + blockIdx.y;  // 0: N_g (values, zero start); 1: M_g (identity start)
    }
    const bool has_v = OUT || part == 0;
    const bf16_t* kh = k + (long)head * T * DK;
    const bf16_t* qh = q + (long)head * T * DK;
    const bf16_t* vh = v + (long)head * T * NS;
    const bf16_t* bh = beta + (long)head * T;

    // state tiles owned by this wave: row tile xrt, column tiles xc0 .. xc0+X_CPW-1
    const int xrt = w % Y::XR, xc0 = (w / Y::XR) * Y::X_CPW;
    // C x NS tiles owned by this wave: row tile ort, column tiles oc0 ..
    const int ort = w % 4, oc0 = (w / 4) * Y::O_CPW;

    v4f X[Y::X_CPW];
#pragma unroll
    for (int c = 0; c < Y::X_CPW; ++c) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * xrt + 4 * g + r, col = 16 * (xc0 + c) + li;
            float x = 0.f;
            if constexpr (OUT) {
                x = state_in[((long)(head * G + seg) * DK + row) * NS + col];
            } else {
                if (part == 1) x = (row == col) ? 1.f : 0.f;
            }
            X[c][r] = x;
        }
    }

    const int t_end = min((seg + 1) * L, T);
    // The next chunk's rows are loaded into registers while this one is
    // processed; rows past the segment end load as zero.
    ChunkRegs<bf16_t, DK, NT> kr, qr;
    ChunkRegs<bf16_t, NS, NT> vr;
    float bnext = 0.f;
    auto load_chunk = [&](int c) {
        const int nn = min(CH, t_end - c);
        kr.load(kh, c, nn, tid);
        if constexpr (OUT) qr.load(qh, c, nn, tid);
        if (has_v) vr.load(vh, c, nn, tid);
        if (tid < CH) bnext = tid < nn ? bf16_to_f32(bh[c + tid]) : 0.f;
    };
    load_chunk(seg * L);
    for (int c0 = seg * L; c0 < t_end; c0 += CH) {
        const int n = min(CH, t_end - c0);
        // ---- stage the chunk (row-major; transposed operands are read with
        // transpose loads); the state goes to LDS as bf16, transposed
        stage_rows_raw<bf16_t, DK, NT>(kr, tid, Ks, LQ);
        if constexpr (OUT) stage_rows_raw<bf16_t, DK, NT>(qr, tid, Qs, LQ);
        if (has_v) stage_rows_raw<bf16_t, NS, NT>(vr, tid, Vs, LV);
        if (tid < CH) Bs[tid] = bnext;
        if (c0 + CH < t_end) load_chunk(c0 + CH);
#pragma unroll
        for (int c = 0; c < Y::X_CPW; ++c) {
            __bf16* dst = &Xt[(16 * (xc0 + c) + li) * LQ + 16 * xrt + 4 * g];
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[r] = M::cvt(X[c][r]);
        }
        __syncthreads();

        // ---- A = tril_{-1}(K K^T) diag(beta) into Af (lower tiles only)
#pragma unroll
        for (int rep = 0; rep < 2; ++rep) {
            const int id = w + NWV * rep;
            if (id < 10) {
                int bi, bj;
                lower_tile(id, bi, bj);
                v4f acc = zero4();
#pragma unroll
                for (int kb = 0; kb < DK / 32; ++kb) {
                    const frag a = M::load(&Ks[(16 * bi + li) * LQ + 32 * kb], g);
                    const frag b = M::load(&Ks[(16 * bj + li) * LQ + 32 * kb], g);
                    M::mma(acc, a, b);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * bi + 4 * g + r, i = 16 * bj + li;
                    Af[t * LF + i] = (i < t) ? Bs[i] * acc[r] : 0.f;
                }
            }
        }
        // ---- P^T tiles (keys x this wave's queries) and O = Q S
        v4f Pt[4];
        v4f Oacc[Y::O_CPW];
        if constexpr (OUT) {
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                Pt[kt] = zero4();
                if (kt <= ort) {
#pragma unroll
                    for (int kb = 0; kb < DK / 32; ++kb) {
                        const frag a = M::load(&Ks[(16 * kt + li) * LQ + 32 * kb], g);
                        const frag b = M::load(&Qs[(16 * ort + li) * LQ + 32 * kb], g);
                        M::mma(Pt[kt], a, b);
                    }
                    if (kt == ort) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (4 * g + r > li) Pt[kt][r] = 0.f;
                    }
                }
            }
#pragma unroll
            for (int c = 0; c < Y::O_CPW; ++c) {
                Oacc[c] = zero4();
#pragma unroll
                for (int kb = 0; kb < DK / 32; ++kb) {
                    const frag a = M::load(&Qs[(16 * ort + li) * LQ + 32 * kb], g);
                    const frag b = M::load(&Xt[(16 * (oc0 + c) + li) * LQ + 32 * kb], g);
                    M::mma(Oacc[c], a, b);
                }
            }
        }
        __syncthreads();

        // ---- diagonal blocks of T: (I + A_bb)^{-1} by forward substitution.
        // Wave 0, lane 16b+j holds column j of block b in registers.
        if (w == 0) {
            const int b = g, j = li;
            float d[16];
#pragma unroll
            for (int m = 0; m < 16; ++m) d[m] = (m == j) ? 1.f : 0.f;
#pragma unroll
            for (int i = 1; i < 16; ++i) {
                const float* arow = &Af[(16 * b + i) * LF + 16 * b];
                float s = 0.f;
#pragma unroll
                for (int m = 0; m < i; ++m) s += arow[m] * d[m];
                if (i > j) d[i] = -s;
            }
#pragma unroll
            for (int m = 0; m < 16; ++m) Af[(16 * b + m) * LF + 16 * b + j] = d[m];
        }
        __syncthreads();

        // ---- off-diagonal blocks, by distance from the diagonal.  T_ij
        // (i > j) is stored in the (unused) upper block at rows 16j, cols 16i.
#pragma unroll
        for (int dist = 1; dist < 4; ++dist) {
            if (w >= 1 && w <= 4 - dist) {
                const int j = w - 1, i = j + dist;
                v4f P = zero4();
                for (int m = j; m < i; ++m) {
                    // A_im (lower block) times T_mj (diagonal D_j when m == j,
                    // else the stored block at rows 16j, cols 16m)
                    const v4f a = *reinterpret_cast<const v4f*>(&Af[(16 * i + li) * LF + 16 * m + 4 * g]);
                    v4f bb;
#pragma unroll
                    for (int s = 0; s < 4; ++s) bb[s] = Af[(16 * j + 4 * g + s) * LF + 16 * m + li];
                    MF::mma(P, a, bb);
                }
                v4f Tij = zero4();
                const v4f a = *reinterpret_cast<const v4f*>(&Af[(16 * i + li) * LF + 16 * i + 4 * g]);
                MF::mma(Tij, a, P);  // an output tile is already in B-operand layout
#pragma unroll
                for (int r = 0; r < 4; ++r) Af[(16 * j + 4 * g + r) * LF + 16 * i + li] = -Tij[r];
            }
            __syncthreads();
        }

        // ---- T to bf16, lower triangular, rows t, k = i
        for (int e = tid; e < CH * CH; e += NT) {
            const int t = e / CH, i = e % CH, bt = t / 16, bi = i / 16;
            float x = 0.f;
            if (bt == bi) x = Af[t * LF + i];
            else if (bt > bi) x = Af[(16 * bi + t % 16) * LF + 16 * bt + i % 16];
            Ts[t * LT + i] = M::cvt(x);
        }
        __syncthreads();

        // ---- W = T K (written transposed-computed so rows land as 8-byte
        // stores) and U_v = T V
#pragma unroll
        for (int c = 0; c < Y::W_TPW; ++c) {
            const int dkt = w % Y::XR, tt = (w / Y::XR) * Y::W_TPW + c;
            v4f acc = zero4();
#pragma unroll
            for (int kb = 0; kb < CH / 32; ++kb) {
                const frag a = M::load_tr(Ks, LQ, 32 * kb, 16 * dkt, lane);
                const frag b = M::load(&Ts[(16 * tt + li) * LT + 32 * kb], g);
                M::mma(acc, a, b);
            }
            __bf16* dst = &Ws[(16 * tt + li) * LQ + 16 * dkt + 4 * g];
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[r] = M::cvt(acc[r]);
        }
        v4f U[Y::O_CPW];
#pragma unroll
        for (int c = 0; c < Y::O_CPW; ++c) {
            U[c] = zero4();
            if (has_v) {
#pragma unroll
                for (int kb = 0; kb < CH / 32; ++kb) {
                    if (32 * kb > 16 * ort + 15) continue;  // T is lower triangular
                    const frag a = M::load(&Ts[(16 * ort + li) * LT + 32 * kb], g);
                    const frag b = M::load_tr(Vs, LV, 32 * kb, 16 * (oc0 + c), lane);
                    M::mma(U[c], a, b);
                }
            }
        }
        __syncthreads();

        // ---- U = U_v - W S, then (beta o U)^T to LDS
#pragma unroll
        for (int c = 0; c < Y::O_CPW; ++c) {
            v4f ws_ = zero4();
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                const frag a = M::load(&Ws[(16 * ort + li) * LQ + 32 * kb], g);
                const frag b = M::load(&Xt[(16 * (oc0 + c) + li) * LQ + 32 * kb], g);
                M::mma(ws_, a, b);
            }
            __bf16* dst = &Ut[(16 * (oc0 + c) + li) * LT + 16 * ort + 4 * g];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                U[c][r] -= ws_[r];
                dst[r] = M::cvt(Bs[16 * ort + 4 * g + r] * U[c][r]);
            }
        }
        __syncthreads();

        // ---- S += K^T (beta o U);  O = Q S + tril(Q K^T) (beta o U)
#pragma unroll
        for (int c = 0; c < Y::X_CPW; ++c) {
#pragma unroll
            for (int kb = 0; kb < CH / 32; ++kb) {
                const frag a = M::load_tr(Ks, LQ, 32 * kb, 16 * xrt, lane);
                const frag b = M::load(&Ut[(16 * (xc0 + c) + li) * LT + 32 * kb], g);
                M::mma(X[c], a, b);
            }
        }
        if constexpr (OUT) {
            bf16_t* oh = o + ((long)head * T + c0) * NS;
#pragma unroll
            for (int c = 0; c < Y::O_CPW; ++c) {
#pragma unroll
                for (int j = 0; j < CH / 32; ++j) {
                    if (32 * j > 16 * ort + 15) continue;  // keys after these queries
                    const frag a = M::from_tiles(Pt[2 * j], Pt[2 * j + 1]);
                    const frag b = M::load(&Ut[(16 * (oc0 + c) + li) * LT + 32 * j], g);
                    M::mma(Oacc[c], a, b);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * ort + 4 * g + r;
                    if (t < n) oh[(long)t * NS + 16 * (oc0 + c) + li] = f32_to_bf16(Oacc[c][r]);
                }
            }
        }
        __syncthreads();
    }

    float* dst = nullptr;
    if constexpr (OUT) {
        if (seg == G - 1 && S_out) dst = S_out + (long)head * DK * NS;
    } else {
        dst = (part == 0 ? map_n : map_m) + (long)(head * G + seg) * DK * NS;
    }
    if (dst) {
#pragma unroll
        for (int c = 0; c < Y::X_CPW; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst[(16 * xrt + 4 * g + r) * NS + 16 * (xc0 + c) + li] = X[c][r];
    }
}

// S_in(0) = S0 (or 0); S_in(g+1) = M_g S_in(g) + N_g in fp32 MFMA.  One
// workgroup per (16-column block of the state, head); serial over segments.
template <int DK, int DV>
__global__ __launch_bounds__(256) void delta_compose_kernel(const float* __restrict__ map_n,
                                                            const float* __restrict__ map_m,
                                                            const float* S0, float* __restrict__ state_in,
                                                            int G) {
    constexpr int RPW = DK / 64;  // row tiles per wave
    __shared__ float Sb[DK][17];
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, li = lane & 15;
    const int w = wave_id(tid);
    const int ct = blockIdx.x, head = blockIdx.y, col = 16 * ct + li;
    v4f acc[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int rt = w * RPW + i;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * rt + 4 * g + r;
            const float x = S0 ? S0[((long)head * DK + row) * DV + col] : 0.f;
            acc[i][r] = x;
            Sb[row][li] = x;
            state_in[((long)head * G * DK + row) * DV + col] = x;
        }
    }
    __syncthreads();
    for (int s = 0; s + 1 < G; ++s) {
        const float* Mg = map_m + (long)(head * G + s) * DK * DK;
        const float* Ng = map_n + (long)(head * G + s) * DK * DV;
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int rt = w * RPW + i;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][r] = Ng[(16 * rt + 4 * g + r) * DV + col];
        }
#pragma unroll 4
        for (int kb = 0; kb < DK / 16; ++kb) {
            v4f b;
#pragma unroll
            for (int e = 0; e < 4; ++e) b[e] = Sb[16 * kb + 4 * g + e][li];
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                const int rt = w * RPW + i;
                const v4f a = *reinterpret_cast<const v4f*>(&Mg[(16 * rt + li) * DK + 16 * kb + 4 * g]);
                Mma<float>::mma(acc[i], a, b);
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int rt = w * RPW + i;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * rt + 4 * g + r;
                Sb[row][li] = acc[i][r];
                state_in[(((long)head * G + s + 1) * DK + row) * DV + col] = acc[i][r];
            }
        }
        __syncthreads();
    }
}

template <int DK, int DV>
hipError_t launch_typed(const bf16_t* q, const bf16_t* k, const bf16_t* v, const bf16_t* beta,
                        const float* S0, bf16_t* o, float* S_out, int HT, int T, const LaPlan& plan,
                        float* ws, hipStream_t stream) {
    const int G = plan.G, L = plan.L;
    float* map_n = ws;
    float* map_m = map_n + (size_t)HT * G * DK * DV;
    float* state_in = map_m + (size_t)HT * G * DK * DK;
    hipError_t err;
    if (G > 1) {
        if constexpr (DK == DV) {
            delta_chunk_kernel<DK, DK, false><<<dim3(HT * (G - 1), 2), dim3(NT), 0, stream>>>(
                q, k, v, beta, nullptr, nullptr, map_n, map_m, nullptr, T, L, G, 0);
        } else {
            delta_chunk_kernel<DK, DV, false><<<dim3(HT * (G - 1), 1), dim3(NT), 0, stream>>>(
                q, k, v, beta, nullptr, nullptr, map_n, map_m, nullptr, T, L, G, 0);
            if ((err = hipGetLastError()) != hipSuccess) return err;
            delta_chunk_kernel<DK, DK, false><<<dim3(HT * (G - 1), 1), dim3(NT), 0, stream>>>(
                q, k, v, beta, nullptr, nullptr, map_n, map_m, nullptr, T, L, G, 1);
        }
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    delta_compose_kernel<DK, DV><<<dim3(DV / 16, HT), dim3(256), 0, stream>>>(map_n, map_m, S0, state_in, G);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    delta_chunk_kernel<DK, DV, true><<<dim3(HT * G), dim3(NT), 0, stream>>>(
        q, k, v, beta, o, state_in, nullptr, nullptr, S_out, T, L, G, 0);
    return hipGetLastError();
}

}  // namespace

size_t delta_ws_floats(int HT, int dk, int dv, const LaPlan& plan) {
    return (size_t)HT * plan.G * ((size_t)dk * dv + (size_t)dk * dk + (size_t)dk * dv);
}

hipError_t launch_delta_forward(const void* q, const void* k, const void* v, const void* beta,
                                const float* S0, void* o, float* S_out, int HT, int T, int dk, int dv,
                                int dtype, const LaPlan& plan, float* ws, hipStream_t stream) {
    if (dtype != 1) return hipErrorInvalidValue;
    const bf16_t* qb = static_cast<const bf16_t*>(q);
    const bf16_t* kb = static_cast<const bf16_t*>(k);
    const bf16_t* vb = static_cast<const bf16_t*>(v);
    const bf16_t* bb = static_cast<const bf16_t*>(beta);
    bf16_t* ob = static_cast<bf16_t*>(o);
#define DELTA_CASE(A, B) \
    if (dk == A && dv == B) return launch_typed<A, B>(qb, kb, vb, bb, S0, ob, S_out, HT, T, plan, ws, stream);
    DELTA_CASE(64, 64)
    DELTA_CASE(64, 128)
    DELTA_CASE(128, 64)
    DELTA_CASE(128, 128)
#undef DELTA_CASE
    return hipErrorInvalidValue;
}

}  // namespace la
