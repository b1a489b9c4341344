// Segment prefix of a packed batch, built on the device from the sequence
// offsets (see segments.hpp): sp[0] = 0, sp[n+1] = sp[n] + ceil(len(n) / L).
// One workgroup walks the sequences in tiles of 1024 with a block scan.
#include "common.hpp"
#include "kernels.hpp"

namespace la {

namespace {

constexpr int NT = 1024;

__global__ __launch_bounds__(NT) void segment_prefix_kernel(const int* __restrict__ cu, int N, int T_total, int L,
                                                            int* __restrict__ sp) {
    __shared__ int wave_sum[NT / 64];
    __shared__ int carry;
    SegMap sm{};
    sm.cu = cu;
    sm.N = N;
    sm.T = T_total;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (tid == 0) {
        carry = 0;
        sp[0] = 0;
    }
    __syncthreads();
    for (int base = 0; base < N; base += NT) {
        const int n = base + tid;
        int x = n < N ? (sm.length<true>(n) + L - 1) / L : 0;
        // inclusive scan: within the wave, then across the waves' totals
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off);
            x += lane >= off ? y : 0;
        }
        if (lane == 63) wave_sum[w] = x;
        __syncthreads();
        int before = carry;
        for (int u = 0; u < w; ++u) before += wave_sum[u];
        if (n < N) sp[n + 1] = before + x;
        __syncthreads();
        if (tid == NT - 1) carry = before + x;
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_segment_prefix(const int* cu, int N, int T_total, int L, int* sp, hipStream_t stream) {
    segment_prefix_kernel<<<dim3(1), dim3(NT), 0, stream>>>(cu, N, T_total, L, sp);
    return hipGetLastError();
}

}  // namespace la
