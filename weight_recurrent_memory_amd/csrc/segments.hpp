// How a prefill call's tokens are cut into (head, sequence, segment) units.
//
// Two batch layouts share one description:
//   uniform  q [B][H][T][d]: sequence n = batch row n, every sequence T tokens;
//   packed   q [H][T_total][d] with sequence offsets cu[0..N] (cu[0] = 0,
//            cu[N] = T_total): sequence n is rows cu[n] .. cu[n+1]-1 of every
//            head, and each sequence starts from its own initial state (the
//            per-request reset of "AIGC 基本功｜线性、循环与记忆架构-LinearMem" §05;
//            "手撕：递推与记忆模型", "验证边界": state reset at request, batch and
//            document boundaries).
// In both, token t of sequence n in head h sits at row h * hs + start(n) + t
// of the input (hs = T uniform, T_total packed; start(n) = n * H * T uniform,
// cu[n] packed), and its initial and final states are entry n * H + h of
// S0 / S_out.  A sequence is cut into segments of L tokens (the last one
// ragged); sp[n] counts the segments of the sequences before n, so the
// segments of all sequences of one head are numbered 0 .. NS - 1, and the
// call has H * NS (head, segment) units in all.
#pragma once
#include <hip/hip_runtime.h>

namespace la {

struct SegMap {
    const int* cu;  // packed: device [N+1] sequence offsets; nullptr: uniform batch
    const int* sp;  // packed: device [N+1] prefix sums of segments per sequence
    int N;          // sequences (uniform: B)
    int H;          // heads
    int T;          // uniform: tokens per sequence; packed: T_total
    int G;          // uniform: segments per sequence
    int L;          // tokens per segment (a multiple of the chunk)
    int NS;         // segments per head, all sequences
    long hs;        // rows between consecutive heads of the input

    // Every accessor takes P = packed() as a template argument, so a uniform
    // batch's kernels compile to plain arithmetic with no offset loads.
    __host__ __device__ bool packed() const { return cu != nullptr; }
    // First row (within a head) and length of sequence n.  Packed offsets are
    // clamped into [0, T], so inconsistent offsets cannot address past the
    // input (they give wrong, not out-of-bounds, results).
    template <bool P>
    __device__ __forceinline__ long start(int n) const {
        if constexpr (!P) {
            return (long)n * H * T;
        } else {
            const int a = cu[n];
            return a < 0 ? 0 : (a > T ? T : a);
        }
    }
    template <bool P>
    __device__ __forceinline__ int length(int n) const {
        if constexpr (!P) {
            return T;
        } else {
            const int a = (int)start<true>(n);
            int b = cu[n + 1];
            b = b < a ? a : (b > T ? T : b);
            return b - a;
        }
    }
    template <bool P>
    __device__ __forceinline__ int seg_base(int n) const {
        if constexpr (!P) return n * G;
        else return sp[n];
    }
    template <bool P>
    __device__ __forceinline__ int segs(int n) const {
        if constexpr (!P) return G;
        else return sp[n + 1] - sp[n];
    }
    // Workspace slot of segment 0 of (sequence n, head h); a sequence's
    // segments occupy consecutive slots.  Uniform batches keep them head by
    // head in batch order ((n H + h) G); packed ones head-major over the
    // global segment numbering (h NS + seg_base(n)).
    template <bool P>
    __device__ __forceinline__ long slot(int n, int h) const {
        if constexpr (!P) return ((long)n * H + h) * G;
        else return (long)h * NS + sp[n];
    }
    // Per-chunk records (one per head, sequence and chunk of C tokens):
    // chunk c of sequence n in head h.  Uniform: (n H + h) ceil(T / C) + c.
    // Packed: h R + floor(start(n) / C) + n + c with R = floor(T / C) + N
    // records per head -- increasing in (n, c) and below R, since
    // floor(a / C) + ceil(b / C) <= floor((a + b) / C) + 1; the gaps between
    // sequences stay unused.
    __host__ __device__ long chunk_recs_per_head(int C) const {
        return packed() ? (long)(T / C + N) : (long)N * ((T + C - 1) / C);
    }
    template <bool P>
    __device__ __forceinline__ long chunk_rec(int n, int h, int c, int C) const {
        if constexpr (!P) return ((long)n * H + h) * ((T + C - 1) / C) + c;
        else return (long)h * (T / C + N) + start<true>(n) / C + n + c;
    }
    // The sequence holding global segment vs (0 <= vs < NS): the largest n
    // with seg_base(n) <= vs.
    template <bool P>
    __device__ __forceinline__ int seq_of(int vs) const {
        if constexpr (!P) {
            return vs / G;
        } else {
            int lo = 0, hi = N - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (sp[mid] <= vs) lo = mid;
                else hi = mid - 1;
            }
            return lo;
        }
    }
    // The sequence holding the i-th segment that is not the last of its
    // sequence (0 <= i < NS - N): the largest n with seg_base(n) - n <= i.
    template <bool P>
    __device__ __forceinline__ int seq_of_inner(int i) const {
        if constexpr (!P) {
            return i / (G - 1);
        } else {
            int lo = 0, hi = N - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (sp[mid] - mid <= i) lo = mid;
                else hi = mid - 1;
            }
            return lo;
        }
    }
};

}  // namespace la
