// Causal ELU+1 linear attention, chunked prefill on gfx950.
//
// The method ("AIGC 基本功｜线性、循环与记忆架构-LinearMem", §03): with
// phi = ELU+1, S_t = S_{t-1} + phi(k_t) v_t^T, z_t = z_{t-1} + phi(k_t) and the
// write-then-read output o_t^T = phi(q_t)^T S_t / (phi(q_t)^T z_t + eps).
//
// Chunked form (a chunk of C = 64 tokens, state (S, z) at the chunk start):
//   P     = tril(phi(Q_c) phi(K_c)^T)                 (diagonal kept: write-then-read)
//   num   = P V_c + phi(Q_c) S,  den = P 1 + phi(Q_c) z + eps,  O_c = num / den
//   S    += phi(K_c)^T V_c,      z  += phi(K_c)^T 1
// Only the state crosses a chunk boundary ("手撕：递推与记忆模型", "Chunked
// scan"; the chunkwise small-attention-plus-state form of "线性注意力与 SSM"
// §3).  The sum z rides along as one extra 16-column tile: V is extended with
// a block of ones and S with 16 copies of z, so the denominator comes out of
// the same MFMA chain as the numerator, in the same registers.
//
// Sequence parallelism: the tokens of each (sequence, head) are cut into
// segments, one workgroup each.  Because the state update is additive, the
// state entering segment g is S0 + sum_{g' < g} (segment sum of g');
// workgroups find it by decoupled look-back over their predecessors'
// published sums (one launch).
// Every flag word carries the tag of the call that wrote it, so flags left
// by earlier calls read as absent and no clearing launch is needed.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace la {

namespace {

constexpr int CH = kChunk;
constexpr int NTHR = 256;  // four waves; wave w owns query rows 16w..16w+15
constexpr unsigned kResidentGroups = 512;  // la_fused workgroups resident at once: two per CU, 256 CUs

template <typename TIn, int DK, int DV>
struct Layout {
    using op = typename Mma<TIn>::op_t;
    static constexpr int PAD = 16 / sizeof(op);
    static constexpr int LQ = DK + PAD;          // rows of phi(Q), phi(K) and S^T: k = dk
    static constexpr int LV = DV + PAD;          // rows of V and of the output tile
    static constexpr int NCT = DV / 16 + 1;      // value column tiles + the ones/z tile
    static constexpr int RTW = DK / 64;          // dk row tiles per wave (4 waves)
    static constexpr int E = DK * DV + DK;       // floats per (head, segment) state
    static constexpr int KSZ = CH * LQ;          // elements of one phi(K) chunk buffer
    static constexpr int VSZ = CH * LV;          // elements of one V chunk buffer
    static constexpr int SSZ = (DV + 16) * LQ;   // elements of one S^T buffer
    static constexpr int bytes(int nst) { return (int)sizeof(op) * (2 * KSZ + 2 * VSZ + nst * SSZ); }
    // S^T is double-buffered (one barrier per chunk) unless that costs a
    // workgroup of residency or does not fit at all.
    static constexpr int kLds = 160 * 1024;
    static constexpr int NST = (2 * bytes(2) <= kLds) ? 2 : (2 * bytes(1) <= kLds) ? 1 : (bytes(2) <= kLds) ? 2 : 1;
    static constexpr int LDS_BYTES = bytes(NST);
};

// ------------------------------------------------------------- la_fused
//
// Single pass with decoupled look-back.  Each workgroup handles one segment
// of one (sequence, head), numbered so that every predecessor segment of the
// same sequence and head has a smaller block index and was dispatched
// earlier (segment-major for a uniform batch; sequence-major for a packed
// one, whose first segment of each sequence starts from that sequence's own
// initial state):
//   1. sum phi(K)^T [V | 1] over its segment (its aggregate);
//   2. publish the aggregate (flag 1); find the state entering the segment by
//      walking back over predecessors: an inclusive state (flag 2) ends the
//      walk, an aggregate is added and the walk continues;
//   3. publish its own inclusive state (flag 2);
//   4. run the chunk loop from that state, writing the outputs.
// Published states are written and read with accesses coherent across the
// chip's L2s; the flag is stored only after the data stores have completed.
// Every wait is bounded (poll_limit polls of one window; a negative limit
// skips the look-back altogether): a workgroup that gives up recomputes its
// incoming state from the inputs, so progress never depends on the dispatch
// order.  It recomputes every predecessor's aggregate with the routine that
// predecessor used and adds them to S0 left to right -- the same operations
// in the same order as the look-back's sum -- so the result is the same bit
// for bit on either path.

enum : int { kFlagNone = 0, kFlagAggregate = 1, kFlagInclusive = 2 };

// A flag word is (tag << 2) | state; a word with another call's tag is absent.
typedef unsigned long long flag_t;
__device__ __forceinline__ int load_flag(const flag_t* p, flag_t tag) {
    const flag_t f = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return (f >> 2) == tag ? (int)(f & 3) : kFlagNone;
}
__device__ __forceinline__ void store_flag(flag_t* p, flag_t tag, int state) {
    __hip_atomic_store(p, (tag << 2) | (flag_t)state, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Published (head, segment) states use a tile-native layout, so that each
// lane moves its four floats of a 16x16 tile in one 16-byte access: tile
// (wave w, row tile i, value tile c) occupies 256 floats, lane l's four at 4l;
// the z column follows the dk x dv block, four floats per (w, i, lane group).
// The accesses are coherent across the chip's L2s (cache policy sc1: stores
// write through, loads miss any stale line), like the relaxed agent-scope
// atomics that carry the flags.
template <int DK, int DV>
struct Published {
    static constexpr int RTW = DK / 64, NVT = DV / 16, NCT = NVT + 1, E = DK * DV + DK;
    static __device__ __forceinline__ uint32_t tile_off(int w, int i, int c, int lane) {
        return (uint32_t)((((w * RTW + i) * NVT + c) * 256 + lane * 4) * 4);
    }
    static __device__ __forceinline__ uint32_t z_off(int w, int i, int g) {
        return (uint32_t)((DK * DV + (w * RTW + i) * 16 + g * 4) * 4);
    }
    static __device__ __forceinline__ void store(float* base, const v4f (&X)[RTW][NCT], int w, int lane) {
        const rsrc_t rs = make_rsrc(base, E * 4);
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
#pragma unroll
            for (int c = 0; c < NVT; ++c)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, X[i][c]), rs, tile_off(w, i, c, lane), 0,
                                                       /*sc1*/ 16);
            if ((lane & 15) == 0)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, X[i][NCT - 1]), rs,
                                                       z_off(w, i, lane >> 4), 0, /*sc1*/ 16);
        }
    }
    static __device__ __forceinline__ void load(const float* base, v4f (&X)[RTW][NCT], int w, int lane) {
        const rsrc_t rs = make_rsrc(base, E * 4);
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
#pragma unroll
            for (int c = 0; c < NVT; ++c)
                X[i][c] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rs, tile_off(w, i, c, lane), 0, 16));
            X[i][NCT - 1] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rs, z_off(w, i, lane >> 4), 0, 16));
        }
    }
};

// Chunks of keys and values held in flight by the aggregate pass: enough
// bytes outstanding per workgroup to cover the memory latency of a streaming
// reduction.
template <typename TIn, int DK, int DV>
constexpr int kPrefetch = (DK + DV) * (int)sizeof(TIn) <= 256 ? 4 : 2;

// acc += phi(K)^T [V | 1] for the chunk staged in LDS at Ks, Vs.
template <typename TIn, int DK, int DV>
__device__ __forceinline__ void add_staged(const typename Mma<TIn>::op_t* Ks, const typename Mma<TIn>::op_t* Vs,
                                           v4f (&acc)[Layout<TIn, DK, DV>::RTW][Layout<TIn, DK, DV>::NCT],
                                           int lane, int w) {
    using M = Mma<TIn>;
    using LY = Layout<TIn, DK, DV>;
    constexpr int NVT = DV / 16;
#pragma unroll
    for (int j = 0; j < CH / M::KB; ++j) {
#pragma unroll
        for (int i = 0; i < LY::RTW; ++i) {
            const typename M::frag a = M::load_tr(Ks, LY::LQ, j * M::KB, 16 * (w * LY::RTW + i), lane);
#pragma unroll
            for (int c = 0; c < LY::NCT; ++c)
                M::mma(acc[i][c], a, c < NVT ? M::load_tr(Vs, LY::LV, j * M::KB, 16 * c, lane) : M::ones());
        }
    }
}

// The raw key and value rows of a segment's first NPF chunks, kept in
// registers from the aggregate pass to the output pass so that they are read
// from memory once.
template <typename TIn, int DK, int DV>
struct KeptChunks {
    static constexpr int N = kPrefetch<TIn, DK, DV>;
    static constexpr int VGPRS = N * (ChunkRegs<TIn, DK, NTHR>::NV + ChunkRegs<TIn, DV, NTHR>::NV) * 4;
    ChunkRegs<TIn, DK, NTHR> k[N];
    ChunkRegs<TIn, DV, NTHR> v[N];
};

// One more chunk kept, raw, in LDS: chunk N of the segment (the first chunk
// after the register-kept ones), where two workgroups per CU still fit with
// it.  Each thread stores and reloads its own 16-byte pieces, so no barrier
// orders the two.
template <typename TIn, int DK, int DV>
struct LdsKept {
    static constexpr int NVK = ChunkRegs<TIn, DK, NTHR>::NV, NVV = ChunkRegs<TIn, DV, NTHR>::NV;
    static constexpr int BYTES = (NVK + NVV) * NTHR * 16;
    static constexpr bool ON = 2 * (Layout<TIn, DK, DV>::LDS_BYTES + BYTES) <= 160 * 1024;
    static __device__ __forceinline__ void put(uint4* buf, const ChunkRegs<TIn, DK, NTHR>& kr,
                                               const ChunkRegs<TIn, DV, NTHR>& vr, int tid) {
#pragma unroll
        for (int j = 0; j < NVK; ++j) buf[j * NTHR + tid] = kr.r[j];
#pragma unroll
        for (int j = 0; j < NVV; ++j) buf[(NVK + j) * NTHR + tid] = vr.r[j];
    }
    static __device__ __forceinline__ void get(const uint4* buf, ChunkRegs<TIn, DK, NTHR>& kr,
                                               ChunkRegs<TIn, DV, NTHR>& vr, int tid) {
#pragma unroll
        for (int j = 0; j < NVK; ++j) kr.r[j] = buf[j * NTHR + tid];
#pragma unroll
        for (int j = 0; j < NVV; ++j) vr.r[j] = buf[(NVK + j) * NTHR + tid];
    }
};

// The segment's aggregate phi(K)^T [V | 1] over [t0, t1), its groups of NPF
// chunks taken last to first: the group loaded last is the segment's first
// NPF chunks, which stay in `kept`.  NPF chunks are in flight ahead of the
// one being staged and the two LDS chunk buffers alternate, so one barrier
// per chunk suffices; rows at or past t1 read as zero through the buffer
// resources.  The order of the sum is fixed, so results do not depend on
// timing.
template <typename TIn, int DK, int DV, bool KEEP_LAST>
__device__ __forceinline__ void aggregate_keep(const TIn* kh, const TIn* vh, int t0, int t1,
                                               v4f (&acc)[Layout<TIn, DK, DV>::RTW][Layout<TIn, DK, DV>::NCT],
                                               typename Mma<TIn>::op_t* Kb, typename Mma<TIn>::op_t* Vb,
                                               KeptChunks<TIn, DK, DV>& kept, uint4* keep_lds, int tid) {
    using LY = Layout<TIn, DK, DV>;
    constexpr int NPF = KeptChunks<TIn, DK, DV>::N, GS = NPF * CH;
    const int lane = tid & 63, w = wave_id(tid);
    const rsrc_t rk = make_rsrc(kh, (uint32_t)t1 * DK * sizeof(TIn));
    const rsrc_t rv = make_rsrc(vh, (uint32_t)t1 * DV * sizeof(TIn));
    // first chunk of the last group (t0 itself for a segment of at most one
    // group, or an empty one, whose rows all read as zero)
    int c0 = t0 + (t1 - t0 > GS ? (t1 - t0 - 1) / GS * GS : 0);
#pragma unroll
    for (int p = 0; p < NPF; ++p) {
        kept.k[p].load_buf(rk, c0 + p * CH, tid);
        kept.v[p].load_buf(rv, c0 + p * CH, tid);
    }
    auto body = [&](auto slot, auto reload, int c) {
        constexpr int sl = decltype(slot)::value, b = sl & 1;
        typename Mma<TIn>::op_t* Ks = Kb + b * LY::KSZ;
        typename Mma<TIn>::op_t* Vs = Vb + b * LY::VSZ;
        stage_rows_phi<TIn, DK, NTHR>(kept.k[sl], t1 - c, tid, Ks, LY::LQ);
        stage_rows_raw<TIn, DV, NTHR>(kept.v[sl], tid, Vs, LY::LV);
        if constexpr (LdsKept<TIn, DK, DV>::ON && sl == 0 && decltype(reload)::value) {
            if (c == t0 + GS) LdsKept<TIn, DK, DV>::put(keep_lds, kept.k[0], kept.v[0], tid);
        }
        if constexpr (decltype(reload)::value) {
            if (KEEP_LAST && c - GS < t0 + GS) {  // the kept first group: its last read from memory
                kept.k[sl].template load_buf<kLastUse>(rk, c - GS, tid);
                kept.v[sl].template load_buf<kLastUse>(rv, c - GS, tid);
            } else {
                kept.k[sl].load_buf(rk, c - GS, tid);
                kept.v[sl].load_buf(rv, c - GS, tid);
            }
        }
        __syncthreads();
        add_staged<TIn, DK, DV>(Ks, Vs, acc, lane, w);
    };
    auto group = [&](auto reload, int cg) {
        body(std::integral_constant<int, 0>{}, reload, cg);
        body(std::integral_constant<int, 1>{}, reload, cg + CH);
        if constexpr (NPF == 4) {
            body(std::integral_constant<int, 2>{}, reload, cg + 2 * CH);
            body(std::integral_constant<int, 3>{}, reload, cg + 3 * CH);
        }
    };
    for (; c0 > t0; c0 -= GS) group(std::true_type{}, c0);
    group(std::false_type{}, t0);
    __syncthreads();  // the caller reuses the buffers
}

// The same sum as aggregate_keep -- the same chunks, staged the same way and
// added in the same order, so the result is the same bit for bit -- with one
// chunk in flight and nothing kept: for the look-back's give-up path, which
// recomputes predecessors' aggregates and must not add register pressure.
template <typename TIn, int DK, int DV>
__device__ __forceinline__ void aggregate_again(const TIn* kh, const TIn* vh, int t0, int t1,
                                                v4f (&acc)[Layout<TIn, DK, DV>::RTW][Layout<TIn, DK, DV>::NCT],
                                                typename Mma<TIn>::op_t* Kb, typename Mma<TIn>::op_t* Vb, int tid) {
    using LY = Layout<TIn, DK, DV>;
    constexpr int NPF = KeptChunks<TIn, DK, DV>::N, GS = NPF * CH;
    const int lane = tid & 63, w = wave_id(tid);
    const rsrc_t rk = make_rsrc(kh, (uint32_t)t1 * DK * sizeof(TIn));
    const rsrc_t rv = make_rsrc(vh, (uint32_t)t1 * DV * sizeof(TIn));
    const int last = t0 + (t1 - t0 > GS ? (t1 - t0 - 1) / GS * GS : 0);
    for (int cg = last; cg >= t0; cg -= GS) {
        for (int p = 0; p < NPF; ++p) {
            const int c = cg + p * CH;
            ChunkRegs<TIn, DK, NTHR> kr;
            ChunkRegs<TIn, DV, NTHR> vr;
            kr.load_buf(rk, c, tid);
            vr.load_buf(rv, c, tid);
            stage_rows_phi<TIn, DK, NTHR>(kr, t1 - c, tid, Kb, LY::LQ);
            stage_rows_raw<TIn, DV, NTHR>(vr, tid, Vb, LY::LV);
            __syncthreads();
            add_staged<TIn, DK, DV>(Kb, Vb, acc, lane, w);
            __syncthreads();
        }
    }
}

// Registers of one output-pass chunk in flight: phi(K) and V rows for the
// LDS staging, and this wave's raw query fragments (rows 16w + lane % 16).
// These are the last reads of the rows; CP is their cache policy.
template <typename TIn, int DK, int DV, int CP = 0>
struct OutChunk {
    static constexpr int QF = DK / Mma<TIn>::KB;
    ChunkRegs<TIn, DK, NTHR> kr;
    ChunkRegs<TIn, DV, NTHR> vr;
    v4u qraw[QF];
    __device__ __forceinline__ void load(rsrc_t rq, rsrc_t rk, rsrc_t rv, int c0, int w, int tid) {
        constexpr int KB = Mma<TIn>::KB;
        const int lane = tid & 63, g = lane >> 4, li = lane & 15;
        kr.template load_buf<CP>(rk, c0, tid);
        vr.template load_buf<CP>(rv, c0, tid);
        load_q(rq, c0, w, tid);
    }
    __device__ __forceinline__ void load_q(rsrc_t rq, int c0, int w, int tid) {
        constexpr int KB = Mma<TIn>::KB;
        const int lane = tid & 63, g = lane >> 4, li = lane & 15;
#pragma unroll
        for (int kk = 0; kk < QF; ++kk)
            qraw[kk] = buf_load16_cp<CP>(rq, (uint32_t)(((c0 + 16 * w + li) * DK + kk * KB + g * (KB / 4)) * (int)sizeof(TIn)));
    }
};

// ------------------------------------------------------------- output pass
//
// The chunk loop of one wave (W = its index, a compile-time constant so the
// body is straight-line code).  Wave W owns query rows 16W..16W+15 of every
// chunk and dk rows 16 W RTW .. of the state.  Per chunk (state S entering it):
//   P^T  = phi(K) phi(Q_W)^T, keys > query zeroed          (16x16 tiles)
//   N^T  = [V | 1]^T P^T + [S | z]^T phi(Q_W)^T            (transposed outputs)
//   O_W  = N^T / den, stored straight from registers
//   S   += phi(K)^T [V | 1]                                  (this wave's rows)
// phi(Q_W) fragments come from global memory in registers; phi(K), V and the
// bf16 copy of S^T are shared through LDS.  The LDS chunk buffers are double
// buffered: while the matrix cores work on chunk c, the same instruction
// stream stages chunk c + 1 (its loads were issued one chunk earlier) and
// issues the loads of chunk c + 2, so one barrier per chunk suffices.  The
// segment's first chunks take their keys and values from `kept` (only their
// queries are loaded); `in` arrives holding the first chunk's queries.
template <typename TIn, int DK, int DV, int W, int CP>
__device__ __forceinline__ void output_pass(rsrc_t rq, rsrc_t rk, rsrc_t rv, rsrc_t ro, int t_beg, int t_end,
                                            float eps, v4f (&S)[Layout<TIn, DK, DV>::RTW][Layout<TIn, DK, DV>::NCT],
                                            const KeptChunks<TIn, DK, DV>& kept, const uint4* keep_lds,
                                            OutChunk<TIn, DK, DV, CP>& in, typename Mma<TIn>::op_t* lds, int tid) {
    using M = Mma<TIn>;
    using op = typename M::op_t;
    using frag = typename M::frag;
    using LY = Layout<TIn, DK, DV>;
    constexpr int LQ = LY::LQ, LV = LY::LV, NCT = LY::NCT, RTW = LY::RTW, NST = LY::NST;
    constexpr int NVT = DV / 16;            // value column tiles
    constexpr int KB = M::KB;               // contraction per fragment
    constexpr int KT = KB / 16;             // 16-row tiles per fragment
    constexpr int QF = DK / KB;             // phi(Q) fragments per lane
    constexpr int NJ = W / KT + 1;          // key fragments reaching query block W
    constexpr int NJC = CH / KB;            // key fragments per chunk
    constexpr int SZ = (int)sizeof(TIn);
    constexpr int NK = KeptChunks<TIn, DK, DV>::N;  // chunks kept from the aggregate pass
    // V^T fragments are kept for the state update when they fit in 32 VGPRs.
    constexpr bool kKeepV = NVT * NJC * (int)(sizeof(frag) / 4) <= 32;
    const int lane = tid & 63, g = lane >> 4, li = lane & 15;
    op* Kb = lds;
    op* Vb = lds + 2 * LY::KSZ;
    op* Sb = Vb + 2 * LY::VSZ;

    frag qf[2][QF];
    auto write_st = [&](op* st) {
#pragma unroll
        for (int i = 0; i < RTW; ++i)
#pragma unroll
            for (int c = 0; c < NCT; ++c) {
                op* dst = &st[(16 * c + li) * LQ + 16 * (W * RTW + i) + 4 * g];
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[r] = M::cvt(S[i][c][r]);
            }
    };
    // Stage chunk c0 (keys and values kr, vr and the queries of `in`, all in
    // registers) into buffer set b.
    auto stage = [&](auto bconst, int c0, const ChunkRegs<TIn, DK, NTHR>& kr, const ChunkRegs<TIn, DV, NTHR>& vr) {
        constexpr int b = decltype(bconst)::value;
        stage_rows_phi<TIn, DK, NTHR>(kr, t_end - c0, tid, Kb + b * LY::KSZ, LQ);
        stage_rows_raw<TIn, DV, NTHR>(vr, tid, Vb + b * LY::VSZ, LV);
#pragma unroll
        for (int kk = 0; kk < QF; ++kk) qf[b][kk] = M::phi_frag(in.qraw[kk]);
    };
    // Loads of segment chunk n (starting at c0): queries only while it is kept
    // (chunk NK: keys and values from the LDS keep, which holds them when the
    // segment reaches that chunk).
    auto load_chunk = [&](auto nconst, int c0) {
        constexpr int nn = decltype(nconst)::value;
        if constexpr (nn < NK) {
            in.load_q(rq, c0, W, tid);
        } else if constexpr (nn == NK && LdsKept<TIn, DK, DV>::ON) {
            in.load_q(rq, c0, W, tid);
            if (c0 < t_end) {
                LdsKept<TIn, DK, DV>::get(keep_lds, in.kr, in.vr, tid);
            } else {
#pragma unroll
                for (int j = 0; j < LdsKept<TIn, DK, DV>::NVK; ++j) in.kr.r[j] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
                for (int j = 0; j < LdsKept<TIn, DK, DV>::NVV; ++j) in.vr.r[j] = make_uint4(0u, 0u, 0u, 0u);
            }
        } else {
            in.load(rq, rk, rv, c0, W, tid);
        }
    };

    // prologue: chunk 0 staged, chunk 1 in flight
    stage(std::integral_constant<int, 0>{}, t_beg, kept.k[0], kept.v[0]);
    write_st(Sb);
    load_chunk(std::integral_constant<int, 1>{}, t_beg + CH);
    __syncthreads();

    // One chunk; n is the segment index of the next chunk when that is a kept
    // one (n < NK), else NK.
    auto iter = [&](auto bconst, auto nconst, int c0) {
        constexpr int b = decltype(bconst)::value;
        constexpr int n = decltype(nconst)::value;
        const op* Kc = Kb + b * LY::KSZ;
        const op* Vc = Vb + b * LY::VSZ;
        const op* Sc = Sb + (NST == 2 ? b : 0) * LY::SSZ;

        // P^T tiles: keys 16kb.. x this wave's queries
        v4f Pt[W + 1];
#pragma unroll
        for (int kb = 0; kb <= W; ++kb) {
            Pt[kb] = zero4();
#pragma unroll
            for (int kk = 0; kk < QF; ++kk)
                M::mma(Pt[kb], M::load16(&Kc[(16 * kb + li) * LQ + kk * KB], g), qf[b][kk]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (4 * g + r > li) Pt[W][r] = 0.f;
        frag pf[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            pf[j] = M::from_tiles(Pt[KT * j], (KT * j + 1 <= W) ? Pt[(KT * j + 1) <= W ? KT * j + 1 : W] : zero4());

        frag vf[kKeepV ? NVT : 1][NJC];
        if constexpr (kKeepV) {
#pragma unroll
            for (int c = 0; c < NVT; ++c)
#pragma unroll
                for (int j = 0; j < NJC; ++j) vf[c][j] = M::load_tr(Vc, LV, j * KB, 16 * c, lane);
        }
        auto vfrag = [&](int c, int j) -> frag {
            if constexpr (kKeepV) return vf[c][j];
            else return M::load_tr(Vc, LV, j * KB, 16 * c, lane);
        };

        // denominator: 1^T P^T + z^T phi(Q)^T (all 16 rows of the tile equal)
        v4f D = zero4();
#pragma unroll
        for (int j = 0; j < NJ; ++j) M::mma(D, M::ones(), pf[j]);
#pragma unroll
        for (int kk = 0; kk < QF; ++kk) M::mma(D, M::load16(&Sc[(DV + li) * LQ + kk * KB], g), qf[b][kk]);
        const float inv = fast_rcp(D[0] + eps);

        // numerator tiles, normalised and stored from registers
        const int orow = c0 + 16 * W + li;
        auto num_tile = [&](int c) {
            v4f N = zero4();
#pragma unroll
            for (int j = 0; j < NJ; ++j) M::mma(N, vfrag(c, j), pf[j]);
#pragma unroll
            for (int kk = 0; kk < QF; ++kk) M::mma(N, M::load16(&Sc[(16 * c + li) * LQ + kk * KB], g), qf[b][kk]);
            return N * inv;
        };
        if constexpr (SZ == 2) {
            // Tiles c, c+1: lane holds columns 4g..4g+3 of each for query li.
            // One row-pair swap gives every lane 8 consecutive columns:
            // even groups columns 16c + 8(g/2).., odd groups 16(c+1) + 8(g/2)..
#pragma unroll
            for (int c = 0; c < NVT; c += 2) {
                const v4f n0 = num_tile(c), n1 = num_tile(c + 1);
                uint32_t a0 = pack_bf16x2(n0[0], n0[1]), a1 = pack_bf16x2(n0[2], n0[3]);
                uint32_t b0 = pack_bf16x2(n1[0], n1[1]), b1 = pack_bf16x2(n1[2], n1[3]);
                const auto s0 = __builtin_amdgcn_permlane16_swap(a0, b0, false, false);
                const auto s1 = __builtin_amdgcn_permlane16_swap(a1, b1, false, false);
                const v4u x = v4u{(uint32_t)s0[0], (uint32_t)s1[0], (uint32_t)s0[1], (uint32_t)s1[1]};
                const int col = 16 * c + 16 * (g & 1) + 8 * (g >> 1);
                buf_store16_stream(ro, (uint32_t)((orow * DV + col) * SZ), x);
            }
        } else {
#pragma unroll
            for (int c = 0; c < NVT; ++c) {
                const v4f n = num_tile(c);
                buf_store16_stream(ro, (uint32_t)((orow * DV + 16 * c + 4 * g) * SZ),
                               v4u{__float_as_uint(n[0]), __float_as_uint(n[1]), __float_as_uint(n[2]),
                                   __float_as_uint(n[3])});
            }
        }

        // state update with this chunk (this wave's dk rows)
#pragma unroll
        for (int j = 0; j < NJC; ++j)
#pragma unroll
            for (int i = 0; i < RTW; ++i) {
                const frag a = M::load_tr(Kc, LQ, j * KB, 16 * (W * RTW + i), lane);
#pragma unroll
                for (int c = 0; c < NCT; ++c) M::mma(S[i][c], a, c < NVT ? vfrag(c, j) : M::ones());
            }

        // next chunk: stage it, start the one after (reads past the segment
        // end return zero without memory traffic)
        if constexpr (n < NK) stage(std::integral_constant<int, b ^ 1>{}, c0 + CH, kept.k[n], kept.v[n]);
        else stage(std::integral_constant<int, b ^ 1>{}, c0 + CH, in.kr, in.vr);
        load_chunk(std::integral_constant<int, n + 1>{}, c0 + 2 * CH);
        if constexpr (NST == 1) __syncthreads();  // all reads of S^T done
        write_st(Sb + (NST == 2 ? (b ^ 1) : 0) * LY::SSZ);
        __syncthreads();
    };
    // The kept chunks (run whatever the segment's length), then pairs of
    // chunks with no exit between them, so the wait counts stay exact across
    // the back edge; a chunk past t_end reads zeros, adds nothing to the
    // state and has its stores dropped.
    iter(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{}, t_beg);
    iter(std::integral_constant<int, 1>{}, std::integral_constant<int, 2>{}, t_beg + CH);
    if constexpr (NK == 4) {
        iter(std::integral_constant<int, 0>{}, std::integral_constant<int, 3>{}, t_beg + 2 * CH);
        iter(std::integral_constant<int, 1>{}, std::integral_constant<int, 4>{}, t_beg + 3 * CH);
    }
    for (int c0 = t_beg + NK * CH; c0 < t_end; c0 += 2 * CH) {
        iter(std::integral_constant<int, 0>{}, std::integral_constant<int, NK>{}, c0);
        iter(std::integral_constant<int, 1>{}, std::integral_constant<int, NK>{}, c0 + CH);
    }
}

// Cache policy of last reads (POL): 0 default; 1 the output pass's loads
// (the last reads of q, and of the keys and values not kept from the
// aggregate pass) non-temporal; 2 also the aggregate pass's loads of the
// chunks it keeps.
template <typename TIn, int DK, int DV, bool PACKED, int POL>
__global__ __launch_bounds__(NTHR) void la_fused_kernel(const TIn* __restrict__ q,
                                                        const TIn* __restrict__ k,
                                                        const TIn* __restrict__ v,
                                                        const float* S0, const float* z0,
                                                        TIn* __restrict__ o, float* S_out, float* z_out,
                                                        flag_t* __restrict__ flags, flag_t tag, float* __restrict__ agg,
                                                        float* __restrict__ incl, SegMap sm, float eps,
                                                        int poll_limit) {
    using M = Mma<TIn>;
    using op = typename M::op_t;
    using LY = Layout<TIn, DK, DV>;
    constexpr int NCT = LY::NCT, RTW = LY::RTW, E = LY::E;
    __shared__ __align__(16) op lds[LY::LDS_BYTES / sizeof(op)];
    op* Kb = lds;                    // the two phi(K) chunk buffers, then the two V buffers
    op* Vb = lds + 2 * LY::KSZ;
    __shared__ int lb_count, lb_timeout;   // look-back result (wave 0 -> block)
    __shared__ uint4 keep_lds[LdsKept<TIn, DK, DV>::ON ? LdsKept<TIn, DK, DV>::BYTES / 16 : 1];

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, li = lane & 15;
    const int w = wave_id(tid);
    // This workgroup's (head h, sequence nseq, segment seg).  Every
    // predecessor segment of the same sequence and head has a smaller block
    // index: uniform batches are numbered segment-major, packed ones
    // sequence-major with the segments of a sequence consecutive.
    int h, nseq, seg;
    if constexpr (!PACKED) {
        const int HT = sm.N * sm.H, rem = blockIdx.x % HT;
        seg = blockIdx.x / HT;
        nseq = rem / sm.H;
        h = rem % sm.H;
    } else {
        const int vs = blockIdx.x / sm.H;
        h = blockIdx.x % sm.H;
        nseq = sm.seq_of<PACKED>(vs);
        seg = vs - sm.seg_base<PACKED>(nseq);
    }
    const int G = sm.segs<PACKED>(nseq);                        // segments of this sequence
    // Issue priorities.  Uniform batches dispatch segment-major, so about
    // 512 / (N H) consecutive segments of each sequence are resident at once;
    // while computing its aggregate, a segment early in that window runs
    // first (the later ones will wait for its aggregate).  Once it has
    // published, later segments of the sequence (by quarter) run first: they
    // sum more predecessors in the look-back and sit on the critical path.
    // (Measured on B=1 H=32 T=65536: 283.4 -> 274.5 us; the post-publish
    // scheme alone had measured about 3 % before the per-phase split.)
    const int quarter = (4 * seg) / (G > 0 ? G : 1);
    if constexpr (!PACKED) {
        const int win = (int)(kResidentGroups / (unsigned)(sm.N * sm.H));
        const int pos = win >= 4 ? (4 * (seg % win)) / win : 0;  // quarter of the resident window
        if (pos == 0) __builtin_amdgcn_s_setprio(3);
        else if (pos == 1) __builtin_amdgcn_s_setprio(2);
        else if (pos == 2) __builtin_amdgcn_s_setprio(1);
    } else {
        if (quarter >= 3) __builtin_amdgcn_s_setprio(3);
        else if (quarter == 2) __builtin_amdgcn_s_setprio(2);
        else if (quarter == 1) __builtin_amdgcn_s_setprio(1);
    }
    const long head = (long)nseq * sm.H + h;            // index of its states in S0, z0, S_out, z_out
    const long row0 = h * sm.hs + sm.start<PACKED>(nseq);       // first input row of the sequence
    const long sbase = sm.slot<PACKED>(nseq, h);  // workspace slot of its first segment
    const TIn* kh = k + row0 * DK;
    const TIn* vh = v + row0 * DV;
    const int L = sm.L;
    const int len = sm.length<PACKED>(nseq);
    const int t_beg = seg * L, t_end = min((seg + 1) * L, len);
    flag_t* hflags = flags + sbase;

    // element of the (dk x (dv + 1)) state held in tile (i, c), register r
    auto row_of = [&](int i, int r) { return 16 * (w * RTW + i) + 4 * g + r; };
    auto state_index = [&](int i, int c, int r) {
        return c < NCT - 1 ? row_of(i, r) * DV + 16 * c + li : DK * DV + row_of(i, r);
    };

    // ---- 1. this segment's aggregate
    v4f A[RTW][NCT];
#pragma unroll
    for (int i = 0; i < RTW; ++i)
#pragma unroll
        for (int c = 0; c < NCT; ++c) A[i][c] = zero4();
    KeptChunks<TIn, DK, DV> kept;
    aggregate_keep<TIn, DK, DV, POL == 2>(kh, vh, t_beg, t_end, A, Kb, Vb, kept, keep_lds, tid);

    // The first chunk's queries are fetched now, so their latency overlaps
    // the look-back.  Buffer resources end at the segment end: reads
    // past it are zero, writes past it are dropped.
    const rsrc_t rq = make_rsrc(q + row0 * DK, (uint32_t)t_end * DK * sizeof(TIn));
    const rsrc_t rk = make_rsrc(kh, (uint32_t)t_end * DK * sizeof(TIn));
    const rsrc_t rv = make_rsrc(vh, (uint32_t)t_end * DV * sizeof(TIn));
    const rsrc_t ro = make_rsrc(o + row0 * DV, (uint32_t)t_end * DV * sizeof(TIn));
    constexpr int CP = POL >= 1 ? kLastUse : 0;
    OutChunk<TIn, DK, DV, CP> first;
    first.load_q(rq, t_beg, w, tid);

    // ---- 2. publish the aggregate, then walk back for the incoming state
    v4f S[RTW][NCT];
#pragma unroll
    for (int i = 0; i < RTW; ++i)
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int e = state_index(i, c, r);
                float x = 0.f;
                if (c < NCT - 1) { if (S0) x = S0[(long)head * DK * DV + e]; }
                else { if (z0) x = z0[(long)head * DK + (e - DK * DV)]; }
                S[i][c][r] = seg == 0 ? x : 0.f;
            }
    using PUB = Published<DK, DV>;
    if constexpr (!PACKED) {
        if (quarter >= 3) __builtin_amdgcn_s_setprio(3);
        else if (quarter == 2) __builtin_amdgcn_s_setprio(2);
        else if (quarter == 1) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
    }
    if (seg > 0 && seg + 1 < G) {
        PUB::store(agg + (sbase + seg) * E, A, w, lane);
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) store_flag(&hflags[seg], tag, kFlagAggregate);
    }
    if (seg > 0) {
        // Find j*, the nearest predecessor whose inclusive state is published
        // (every segment between j* and this one must have its aggregate
        // out).  Windows of up to 64 predecessors: lane j of wave 0 watches
        // segment base - j.  Segment 0 always publishes an inclusive state,
        // so the walk ends.
        int jstar = -1;
        bool timeout = poll_limit < 0;
        for (int base = seg - 1; base >= 0 && !timeout; base -= 64) {
            if (w == 0) {
                const int p = base - lane;
                int polls = 0, found = -1, to = 0;
                while (true) {
                    const int f = p >= 0 ? load_flag(&hflags[p], tag) : kFlagNone;
                    const unsigned long long incl_mask = __ballot(p >= 0 && f == kFlagInclusive);
                    const unsigned long long ready_mask = __ballot(p < 0 || f != kFlagNone);
                    const int live = __popcll(__ballot(p >= 0));
                    const int stop = incl_mask ? __ffsll((long long)incl_mask) - 1 : 64;
                    const int need = min(stop + 1, live);
                    const unsigned long long need_mask = need >= 64 ? ~0ull : ((1ull << need) - 1);
                    if ((ready_mask & need_mask) == need_mask) {
                        found = incl_mask ? base - stop : -1;
                        break;
                    }
                    if (++polls > poll_limit) {
                        to = 1;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
                if (lane == 0) {
                    lb_count = found;
                    lb_timeout = to;
                }
            }
            __syncthreads();
            // block-uniform values, made visibly uniform (they guard MFMA loops)
            jstar = __builtin_amdgcn_readfirstlane(lb_count);
            timeout = __builtin_amdgcn_readfirstlane(lb_timeout) != 0;
            __syncthreads();
            if (timeout || jstar >= 0) break;
        }
        if (!timeout) {
            // S_in = incl[j*] + agg[j*+1] + ... + agg[seg-1], left to right: the
            // same rounding as the left-to-right sum from S0, whatever j* is,
            // so results do not depend on timing.
            PUB::load(incl + (sbase + jstar) * E, S, w, lane);
            // Aggregates in batches: every load of a batch is issued before
            // the first add, so the walk costs one memory latency per batch.
            // (A batch fits in the registers left beside the kept chunks.)
            constexpr int BUDGET = 160 - KeptChunks<TIn, DK, DV>::VGPRS;
            constexpr int BATCH = BUDGET / (RTW * NCT * 4) >= 8 ? 8 : BUDGET / (RTW * NCT * 4) >= 2 ? BUDGET / (RTW * NCT * 4) : 1;
            for (int p = jstar + 1; p < seg; p += BATCH) {
                v4f t[BATCH][RTW][NCT];
#pragma unroll
                for (int u = 0; u < BATCH; ++u)
                    if (p + u < seg) PUB::load(agg + (sbase + p + u) * E, t[u], w, lane);
#pragma unroll
                for (int u = 0; u < BATCH; ++u)
                    if (p + u < seg) {
#pragma unroll
                        for (int i = 0; i < RTW; ++i)
#pragma unroll
                            for (int c = 0; c < NCT; ++c) S[i][c] += t[u][i][c];
                    }
            }
        } else {
            // Gave up: S_in = S0 + A_0 + ... + A_{seg-1}, left to right, each
            // predecessor aggregate A_j recomputed as segment j computed it
            // (same chunk order, same MFMA chains).  The running sum
            // waits in this segment's own inclusive slot, which no other
            // workgroup reads before this one publishes it (step 3), so that
            // only A_j occupies registers during each recomputation.  S0 is
            // read here while the last segment may already be writing S_out:
            // the host passes a snapshot when the two alias.
#pragma unroll
            for (int i = 0; i < RTW; ++i)
#pragma unroll
                for (int c = 0; c < NCT; ++c)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int e = state_index(i, c, r);
                        float x = 0.f;
                        if (c < NCT - 1) { if (S0) x = S0[(long)head * DK * DV + e]; }
                        else { if (z0) x = z0[(long)head * DK + (e - DK * DV)]; }
                        S[i][c][r] = x;
                    }
            float* run = incl + (sbase + seg) * E;
            PUB::store(run, S, w, lane);
            for (int j = 0; j < seg; ++j) {
#pragma unroll
                for (int i = 0; i < RTW; ++i)
#pragma unroll
                    for (int c = 0; c < NCT; ++c) S[i][c] = zero4();
                aggregate_again<TIn, DK, DV>(kh, vh, j * L, min((j + 1) * L, len), S, Kb, Vb, tid);
                __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the wave's own stores of `run`
                v4f X[RTW][NCT];
                PUB::load(run, X, w, lane);
#pragma unroll
                for (int i = 0; i < RTW; ++i)
#pragma unroll
                    for (int c = 0; c < NCT; ++c) X[i][c] += S[i][c];
                PUB::store(run, X, w, lane);
            }
            __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
            PUB::load(run, S, w, lane);
        }
    }

    // ---- 3. publish the inclusive state (or the final state, last segment)
    if (seg + 1 < G) {
        v4f X[RTW][NCT];
#pragma unroll
        for (int i = 0; i < RTW; ++i)
#pragma unroll
            for (int c = 0; c < NCT; ++c) X[i][c] = S[i][c] + A[i][c];
        PUB::store(incl + (sbase + seg) * E, X, w, lane);
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) store_flag(&hflags[seg], tag, kFlagInclusive);
    } else {
#pragma unroll
        for (int i = 0; i < RTW; ++i)
#pragma unroll
            for (int c = 0; c < NCT; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int e = state_index(i, c, r);
                    const float x = S[i][c][r] + A[i][c][r];
                    if (c < NCT - 1) { if (S_out) S_out[(long)head * DK * DV + e] = x; }
                    else if (li == 0 && z_out) z_out[(long)head * DK + (e - DK * DV)] = x;
                }
    }

    // ---- 4. the chunk loop from the incoming state
    switch (w) {
        case 0: output_pass<TIn, DK, DV, 0, CP>(rq, rk, rv, ro, t_beg, t_end, eps, S, kept, keep_lds, first, lds, tid); break;
        case 1: output_pass<TIn, DK, DV, 1, CP>(rq, rk, rv, ro, t_beg, t_end, eps, S, kept, keep_lds, first, lds, tid); break;
        case 2: output_pass<TIn, DK, DV, 2, CP>(rq, rk, rv, ro, t_beg, t_end, eps, S, kept, keep_lds, first, lds, tid); break;
        default: output_pass<TIn, DK, DV, 3, CP>(rq, rk, rv, ro, t_beg, t_end, eps, S, kept, keep_lds, first, lds, tid); break;
    }
}

// Zeroes the flag words: used where the launch is recorded into a graph, whose
// replays all carry the same tag.
__global__ void la_flags_clear_kernel(flag_t* flags, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) flags[i] = 0;
}

template <typename TIn, int DK, int DV>
hipError_t launch_typed(const void* q, const void* k, const void* v, const float* S0,
                        const float* z0, void* o, float* S_out, float* z_out, const SegMap& sm,
                        float eps, float* ws, unsigned long long tag, bool clear_flags, int poll_limit,
                        hipStream_t stream) {
    const long slots = (long)sm.H * sm.NS;
    flag_t* flags = reinterpret_cast<flag_t*>(ws);
    float* agg = ws + la_flag_words(slots);
    float* incl = agg + (size_t)slots * (DK * DV + DK);
    // In-place continuation (S_out == S0 or z_out == z0) with more than one
    // segment in some sequence: a workgroup that gives up on the look-back
    // reads S0, z0 while the last segment may already have written S_out,
    // z_out, so the kernel reads copies taken before it starts.
    if (sm.NS > sm.N && ((S0 && S0 == S_out) || (z0 && z0 == z_out))) {
        const long states = (long)sm.N * sm.H;
        float* S0c = incl + (size_t)slots * (DK * DV + DK);
        float* z0c = S0c + (size_t)states * DK * DV;
        hipError_t err = hipSuccess;
        if (S0) err = hipMemcpyAsync(S0c, S0, (size_t)states * DK * DV * 4, hipMemcpyDeviceToDevice, stream);
        if (err == hipSuccess && z0)
            err = hipMemcpyAsync(z0c, z0, (size_t)states * DK * 4, hipMemcpyDeviceToDevice, stream);
        if (err != hipSuccess) return err;
        if (S0) S0 = S0c;
        if (z0) z0 = z0c;
    }
    if (clear_flags) {
        la_flags_clear_kernel<<<dim3((unsigned)((slots + 255) / 256)), dim3(256), 0, stream>>>(flags, (int)slots);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    // Last reads non-temporal, so the L2 keeps the keys and values still to
    // be read again -- chosen by measurement (interleaved rounds, per call):
    // uniform batches with every workgroup resident at once (B=4 H=8 T=8192)
    // 44.7 -> 42.2 us with the output pass's loads so marked, the kept
    // chunks' loads too costing 3 %; uniform batches over several rounds
    // (B=1 H=32 T=65536) 275.6 -> 268.5 us with both; the packed serving
    // batch (48 requests, 32768 tokens x 8 heads) 58 -> 62.5 us with both,
    // so packed batches keep the default policy.
    const bool one_round = slots <= (long)kResidentGroups;
    auto kern = sm.packed() ? la_fused_kernel<TIn, DK, DV, true, 0>
                            : (one_round ? la_fused_kernel<TIn, DK, DV, false, 1> : la_fused_kernel<TIn, DK, DV, false, 2>);
    kern<<<dim3((unsigned)slots), dim3(NTHR), 0, stream>>>(
        static_cast<const TIn*>(q), static_cast<const TIn*>(k), static_cast<const TIn*>(v), S0, z0,
        static_cast<TIn*>(o), S_out, z_out, flags, (flag_t)tag, agg, incl, sm, eps, poll_limit);
    return hipGetLastError();
}

}  // namespace

size_t la_flag_words(long slots) { return ((size_t)slots * 2 + 63) / 64 * 64; }  // 64-bit flags, in floats

LaPlan la_plan(int HT, int T, int dk, int dv) {
    // Enough (head, segment) workgroups for two per compute unit, and segments
    // short enough that the keys and values of all resident workgroups (read
    // twice: aggregate, then outputs) stay within the Infinity Cache.  At
    // dk = dv = 64 segments of 12 chunks measured faster than 16 (or 8, 10,
    // 11, 13, 14): five of the chunks are kept, and shorter workgroups leave
    // a shorter tail.
    const int nch = (T + CH - 1) / CH;
    const long occ = ((long)nch * HT) / kResidentGroups;
    const long cap = (dk == 64 && dv == 64) ? 12 : (256L * 1024) / ((long)(dk + dv) * 2 * CH);
    long cps = occ < cap ? occ : cap;
    if (cps < 1) cps = 1;
    LaPlan p;
    p.L = (int)cps * CH;
    p.G = (T + p.L - 1) / p.L;
    return p;
}

size_t la_ws_floats(long slots, long states, int dk, int dv) {
    return la_flag_words(slots) + (size_t)(2 * slots + states) * ((size_t)dk * dv + dk);
}

size_t la_lds_bytes(int dk, int dv, int dtype) {
#define LDS_CASE(TY, DT, A, B) \
    if (dtype == DT && dk == A && dv == B)   \
        return Layout<TY, A, B>::LDS_BYTES + (LdsKept<TY, A, B>::ON ? LdsKept<TY, A, B>::BYTES : 0);
    LDS_CASE(bf16_t, 1, 64, 64)
    LDS_CASE(bf16_t, 1, 64, 128)
    LDS_CASE(bf16_t, 1, 128, 64)
    LDS_CASE(bf16_t, 1, 128, 128)
    LDS_CASE(float, 0, 64, 64)
    LDS_CASE(float, 0, 64, 128)
    LDS_CASE(float, 0, 128, 64)
    LDS_CASE(float, 0, 128, 128)
#undef LDS_CASE
    return (size_t)1 << 30;
}

hipError_t launch_la_forward(const void* q, const void* k, const void* v, const float* S0,
                             const float* z0, void* o, float* S_out, float* z_out, const SegMap& sm,
                             int dk, int dv, int dtype, float eps, float* ws,
                             unsigned long long tag, bool clear_flags, int poll_limit, hipStream_t stream) {
#define LA_CASE(TY, DT, A, B)                                                                                \
    if (dtype == DT && dk == A && dv == B)                                                                   \
        return launch_typed<TY, A, B>(q, k, v, S0, z0, o, S_out, z_out, sm, eps, ws, tag, clear_flags,       \
                                      poll_limit, stream);
    LA_CASE(bf16_t, 1, 64, 64)
    LA_CASE(bf16_t, 1, 64, 128)
    LA_CASE(bf16_t, 1, 128, 64)
    LA_CASE(bf16_t, 1, 128, 128)
    LA_CASE(float, 0, 64, 64)
    LA_CASE(float, 0, 64, 128)
    LA_CASE(float, 0, 128, 64)
#undef LA_CASE
    return hipErrorInvalidValue;
}

}  // namespace la
