// Device helpers shared by the gfx950 kernels: element types, the ELU+1
// feature map, bf16 rounding and 16x16 MFMA fragments.
//
// MFMA fragment convention used by every kernel in this library
// ------------------------------------------------------------
// A 16x16 output tile of v_mfma_f32_16x16x{32_bf16,4_f32} lives in a wave as
// four floats per lane: lane l, register r holds row 4*(l/16)+r, column l%16.
// An A operand supplies, per lane, row l%16; a B operand supplies column l%16;
// each lane group g = l/16 carries a slice of the contraction index.  Which
// logical contraction index sits in which (group, slot) is a free choice as
// long as A and B agree; every kernel here uses the mapping
//     bf16 (k-block of 32):  slot s of group g  <->  k = 4g+s      (s < 4)
//                                                   k = 16+4g+s-4  (s >= 4)
//     f32  (k-block of 16):  MFMA number s, group g  <->  k = 4g+s
// so that the four registers of an output tile (rows 4g..4g+3) are exactly an
// operand slice: an accumulator computed as a transposed tile feeds the next
// contraction without leaving registers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.hpp"

namespace la {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // raw bfloat16 bits in global memory
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- scalars

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even: a plain conversion, which gfx950
// executes as v_cvt_pk_bf16_f32 (NaN stays NaN, no branches).
__device__ __forceinline__ __bf16 f32_to_bf(float f) { return static_cast<__bf16>(f); }
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, f32_to_bf(f)); }
// Two floats -> two bf16 in one 32-bit word (one v_cvt_pk_bf16_f32), a first.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, v2bf{f32_to_bf(a), f32_to_bf(b)});
}

// ELU+1 feature map, "AIGC 基本功｜线性、循环与记忆架构-LinearMem" §03:
// u + 1 for u > 0, e^u otherwise.  e^u is evaluated as 2^(u log2 e) with the
// hardware base-2 exponential (v_exp_f32, about 1 ulp); for u <= 0 the
// result lies in (0, 1] and underflows to 0 below about -87.
__device__ __forceinline__ float phi(float u) {
    return u > 0.f ? u + 1.f : __builtin_amdgcn_exp2f(u * 1.4426950408889634f);
}

// 1/x with the hardware reciprocal (v_rcp_f32, about 1 ulp).
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// ---------------------------------------------------------------- buffers
//
// Raw buffer resources give branch-free edges: a load whose byte offset is
// at or beyond the resource's size returns zero without touching memory, and
// such a store is dropped.  Word 3 selects the 32-bit data format that
// untyped buffer access needs on this architecture family.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufferWord3);
}
__device__ __forceinline__ v4u buf_load16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
// Cache policy of a load: 0 default; kLastUse (non-temporal) for data read
// for the last time, so its lines are the first the L2 gives up.
constexpr int kLastUse = 2;
template <int CP>
__device__ __forceinline__ v4u buf_load16_cp(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CP);
}
// Streaming 16-byte store for results this kernel never reads: non-temporal
// and written through the L2 (cache policy sc1 | nt), so output lines do not
// stay dirty in the L2 beside the input stream.  On the LA prefill this
// measured 44 us per launch against 50 us with the non-temporal hint alone.
constexpr int kStreamWT = 16 | 2;
__device__ __forceinline__ void buf_store16_stream(rsrc_t r, uint32_t off, v4u x) {
    __builtin_amdgcn_raw_buffer_store_b128(x, r, off, 0, kStreamWT);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float* p, long i) { return p[i]; }
    static __device__ __forceinline__ void store(float* p, long i, float x) { p[i] = x; }
};
template <> struct Elem<bf16_t> {
    static __device__ __forceinline__ float load(const bf16_t* p, long i) { return bf16_to_f32(p[i]); }
    static __device__ __forceinline__ void store(bf16_t* p, long i, float x) { p[i] = f32_to_bf16(x); }
};

// ---------------------------------------------------------------- MFMA

// Group-permuted row layout of a bf16 LDS matrix read as row fragments.  A
// fragment gives lane group g the contraction columns 4g..4g+3 and
// 16+4g..16+4g+3 of a 32-column block, two 8-byte pieces 32 bytes apart; on
// gfx950 such paired reads move about half the bytes per clock of one
// 16-byte read per lane and conflict two ways at the 8-element padding.
// Storing the 4-column groups of every 32-column block in the order 0, 4, 1,
// 5, 2, 6, 3, 7 makes the two pieces adjacent: physical column of logical
// column c (whole 4-column groups stay contiguous, so 8-byte stores and
// transpose reads of single groups still work).  With a row stride of D + 16
// elements the 16-byte reads are conflict-free.
__device__ __forceinline__ constexpr int pcol(int c) {
    return (c & ~31) + 4 * (2 * ((c >> 2) & 3) + ((c >> 4) & 1)) + (c & 3);
}


// Operand element type in LDS: bf16 for bf16 inputs, fp32 for fp32 inputs.
template <typename TIn> struct Mma;

template <> struct Mma<bf16_t> {
    typedef __bf16 op_t;          // LDS element
    static constexpr int KB = 32; // contraction per MFMA instruction
    typedef v8bf frag;

    // Fragment from a row of an LDS matrix whose contraction index is
    // contiguous; `row` points at the start of the k-block.
    static __device__ __forceinline__ frag load(const op_t* row, int g) {
        v4bf lo = *reinterpret_cast<const v4bf*>(row + 4 * g);
        v4bf hi = *reinterpret_cast<const v4bf*>(row + 16 + 4 * g);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    // The same fragment from a row stored in the group-permuted layout (pcol
    // below): one 16-byte read.
    static __device__ __forceinline__ frag load_p(const op_t* row, int g) {
        return *reinterpret_cast<const frag*>(row + 8 * g);
    }
    // Fragment whose contraction index runs down the ROWS of a row-major
    // [k][n] LDS matrix (row stride ld elements): rows k0..k0+31, columns
    // n0..n0+15, as an A operand (n = m) or a B operand.  Two gfx950
    // transpose reads: within each 16-lane group, destination lane i, slot s
    // receives element (i & 3) of source lane 4s + (i >> 2); so source lane j
    // of group g points at row k0 + 4g + (j >> 2), columns n0 + 4(j & 3).
    static __device__ __forceinline__ frag load_tr(const op_t* base, int ld, int k0, int n0, int lane) {
        typedef short v4s __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) v4s lds_v4s;
        const int g = lane >> 4, j = lane & 15;
        const op_t* p0 = base + (k0 + 4 * g + (j >> 2)) * ld + n0 + 4 * (j & 3);
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p0));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p0 + 16 * ld));
        return __builtin_bit_cast(frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    static __device__ __forceinline__ frag ones() {
        __bf16 o = __builtin_bit_cast(__bf16, (bf16_t)0x3f80);
        return frag{o, o, o, o, o, o, o, o};
    }
    static __device__ __forceinline__ frag zero() {
        __bf16 o = __builtin_bit_cast(__bf16, (bf16_t)0);
        return frag{o, o, o, o, o, o, o, o};
    }
    // A-operand fragment from two adjacent output tiles (contraction rows
    // 0..15 in t0, 16..31 in t1), scaled elementwise by nothing.
    static __device__ __forceinline__ frag from_tiles(v4f t0, v4f t1) {
        return frag{f32_to_bf(t0[0]), f32_to_bf(t0[1]), f32_to_bf(t0[2]), f32_to_bf(t0[3]),
                    f32_to_bf(t1[0]), f32_to_bf(t1[1]), f32_to_bf(t1[2]), f32_to_bf(t1[3])};
    }
    // The same pair of tiles as two fragments whose sum carries about 16
    // significant bits: hi = bf16(x), lo = bf16(x - hi).  For operands whose
    // products cancel against another term, where one bf16 rounding would
    // set the error of the difference.
    static __device__ __forceinline__ void split_tiles(v4f t0, v4f t1, frag& hi, frag& lo) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            hi[r] = f32_to_bf(t0[r]);
            hi[4 + r] = f32_to_bf(t1[r]);
            lo[r] = f32_to_bf(t0[r] - (float)hi[r]);
            lo[4 + r] = f32_to_bf(t1[r] - (float)hi[4 + r]);
        }
    }
    // Fragment of 16 contiguous bytes: slot s of group g <-> k = 8g + s.  Used
    // where both operands are rows with a contiguous contraction index.
    static __device__ __forceinline__ frag load16(const op_t* row, int g) {
        return *reinterpret_cast<const frag*>(row + 8 * g);
    }
    // phi of 16 raw input bytes (8 bf16) in the load16 slot order.
    static __device__ __forceinline__ frag phi_frag(v4u raw) {
        frag f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t w = raw[e >> 1];
            f[e] = f32_to_bf(phi(__uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16))));
        }
        return f;
    }
    static __device__ __forceinline__ void mma(v4f& acc, const frag& a, const frag& b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
    static __device__ __forceinline__ op_t cvt(float x) { return f32_to_bf(x); }
};

template <> struct Mma<float> {
    typedef float op_t;
    static constexpr int KB = 16;
    typedef v4f frag;
    static __device__ __forceinline__ frag load(const op_t* row, int g) {
        return *reinterpret_cast<const v4f*>(row + 4 * g);
    }
    // Contraction down the rows of a row-major [k][n] matrix: four scalar
    // reads (lane i of group g reads rows k0+4g..k0+4g+3 at column n0+i).
    static __device__ __forceinline__ frag load_tr(const op_t* base, int ld, int k0, int n0, int lane) {
        const int g = lane >> 4, i = lane & 15;
        const op_t* p = base + (k0 + 4 * g) * ld + n0 + i;
        return frag{p[0], p[ld], p[2 * ld], p[3 * ld]};
    }
    static __device__ __forceinline__ frag ones() { return frag{1.f, 1.f, 1.f, 1.f}; }
    static __device__ __forceinline__ frag zero() { return frag{0.f, 0.f, 0.f, 0.f}; }
    static __device__ __forceinline__ frag from_tiles(v4f t0, v4f) { return t0; }
    static __device__ __forceinline__ frag load16(const op_t* row, int g) { return load(row, g); }
    static __device__ __forceinline__ frag phi_frag(v4u raw) {
        return frag{phi(__uint_as_float(raw[0])), phi(__uint_as_float(raw[1])), phi(__uint_as_float(raw[2])),
                    phi(__uint_as_float(raw[3]))};
    }
    static __device__ __forceinline__ void mma(v4f& acc, const frag& a, const frag& b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
    }
    static __device__ __forceinline__ op_t cvt(float x) { return x; }
};

__device__ __forceinline__ v4f zero4() { return v4f{0.f, 0.f, 0.f, 0.f}; }

// Sum over the 16 lanes of each row of the wave (lanes 16r .. 16r + 15), in
// every lane of the row: four DPP adds (quad swaps, then half-row and row
// mirrors), no LDS traffic.  Needs all lanes of the row active.
__device__ __forceinline__ float row16_sum(float x) {
    auto dpp = [](float v, auto ctrl) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), decltype(ctrl)::value,
                                                                  0xF, 0xF, false));
    };
    x += dpp(x, std::integral_constant<int, 0xB1>{});   // quad_perm [1, 0, 3, 2]
    x += dpp(x, std::integral_constant<int, 0x4E>{});   // quad_perm [2, 3, 0, 1]
    x += dpp(x, std::integral_constant<int, 0x141>{});  // row_half_mirror
    x += dpp(x, std::integral_constant<int, 0x140>{});  // row_mirror
    return x;
}

// The wave's index in its workgroup, as a value the compiler knows to be
// uniform across the wave.  MFMA instructions ignore the EXEC mask, so a
// condition guarding an MFMA must compile to a scalar branch that skips it;
// a condition the compiler believes divergent becomes an EXEC-masked block in
// which the MFMA still executes (with stale operands).  Every wave-level
// condition in these kernels derives from this value.
__device__ __forceinline__ int wave_id(int tid) { return __builtin_amdgcn_readfirstlane(tid >> 6); }

// 16-byte global loads of a chunk of rows [c0, c0+n) of a [T][D] matrix.
template <typename TIn, int D, int NT>
struct ChunkRegs {
    static constexpr int VEC = 16 / sizeof(TIn);
    static constexpr int NV = kChunk * D / (NT * VEC);
    static_assert(NV * NT * VEC == kChunk * D, "chunk must split evenly");
    uint4 r[NV];

    __device__ __forceinline__ void load(const TIn* base, int c0, int n, int tid) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int idx = j * NT + tid;
            const int row = idx / (D / VEC);
            const int col = (idx % (D / VEC)) * VEC;
            if (row < n)
                r[j] = *reinterpret_cast<const uint4*>(base + (long)(c0 + row) * D + col);
            else
                r[j] = make_uint4(0u, 0u, 0u, 0u);
        }
    }
    // Same rows through a buffer resource: rows past the resource's end read
    // as zero (no row guard, no branch).
    template <int CP = 0>
    __device__ __forceinline__ void load_buf(rsrc_t rs, int c0, int tid) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int idx = j * NT + tid;
            const int row = idx / (D / VEC);
            const int col = (idx % (D / VEC)) * VEC;
            const v4u x = buf_load16_cp<CP>(rs, (uint32_t)(((c0 + row) * D + col) * (int)sizeof(TIn)));
            r[j] = make_uint4(x[0], x[1], x[2], x[3]);
        }
    }
    static __device__ __forceinline__ int row_of(int j, int tid) { return (j * NT + tid) / (D / VEC); }
    static __device__ __forceinline__ int col_of(int j, int tid) { return ((j * NT + tid) % (D / VEC)) * VEC; }

    __device__ __forceinline__ float get(int j, int e) const {
        const uint32_t w[4] = {r[j].x, r[j].y, r[j].z, r[j].w};
        if constexpr (sizeof(TIn) == 2) {
            const uint32_t x = w[e >> 1];
            return __uint_as_float((e & 1) ? (x & 0xffff0000u) : (x << 16));
        } else {
            return __uint_as_float(w[e]);
        }
    }
};

// Write a staged chunk of the feature-mapped operand into LDS row-major
// ([CH][ld], 16-byte stores).  Rows >= n are stored as zero (not phi(0) = 1)
// by a select, so padding never enters a sum and the code stays one basic
// block.
template <typename TIn, int D, int NT>
__device__ __forceinline__ void stage_rows_phi(const ChunkRegs<TIn, D, NT>& cr, int n, int tid,
                                               typename Mma<TIn>::op_t* rm, int ld) {
    using M = Mma<TIn>;
    using op = typename M::op_t;
    constexpr int VEC = ChunkRegs<TIn, D, NT>::VEC;
#pragma unroll
    for (int j = 0; j < ChunkRegs<TIn, D, NT>::NV; ++j) {
        const int row = ChunkRegs<TIn, D, NT>::row_of(j, tid);
        const int col = ChunkRegs<TIn, D, NT>::col_of(j, tid);
        op vals[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) vals[e] = M::cvt(phi(cr.get(j, e)));
        uint4 x = *reinterpret_cast<const uint4*>(vals);
        const bool keep = row < n;
        x.x = keep ? x.x : 0u;
        x.y = keep ? x.y : 0u;
        x.z = keep ? x.z : 0u;
        x.w = keep ? x.w : 0u;
        *reinterpret_cast<uint4*>(rm + row * ld + col) = x;
    }
}

// Row layout of a bf16 LDS matrix: row stride LD elements, natural or
// group-permuted (pcol).  frag() reads the row fragment of contraction block
// k0 (a multiple of 32) of one row; tr() the transposed fragment of rows
// k0..k0+31, columns n0..n0+15 (n0 a multiple of 16).  Each source lane of
// a transpose read fetches one whole 4-column group, so on permuted rows it
// only points at that group's place; the exchange between lanes is the same.
template <int LD_, bool PERM_ = false>
struct RowLayout {
    static constexpr int LD = LD_;
    static constexpr bool PERM = PERM_;
    static_assert(!PERM || LD % 32 == 16, "permuted rows: 16 elements of padding past a multiple of 32");
    static __device__ __forceinline__ int at(int row, int col) { return row * LD + (PERM ? pcol(col) : col); }
    static __device__ __forceinline__ Mma<bf16_t>::frag frag(const __bf16* X, int row, int k0, int g) {
        if constexpr (PERM) return Mma<bf16_t>::load_p(X + row * LD + k0, g);
        else return Mma<bf16_t>::load(X + row * LD + k0, g);
    }
    static __device__ __forceinline__ Mma<bf16_t>::frag tr(const __bf16* X, int k0, int n0, int lane) {
        if constexpr (!PERM) {
            return Mma<bf16_t>::load_tr(X, LD, k0, n0, lane);
        } else {
            typedef short v4s __attribute__((ext_vector_type(4)));
            typedef __attribute__((address_space(3))) v4s lds_v4s;
            const int g = lane >> 4, j = lane & 15;
            const __bf16* p0 = X + (k0 + 4 * g + (j >> 2)) * LD + pcol(n0 + 4 * (j & 3));
            const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p0));
            const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p0 + 16 * LD));
            return __builtin_bit_cast(Mma<bf16_t>::frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    }
};

// Raw copy of a staged chunk into LDS (operand type == input type).  SPLIT8:
// two 8-byte stores per 16 bytes, for row strides that keep rows only
// 8-byte aligned.  PERM: rows in the group-permuted layout (pcol; bf16).
template <typename TIn, int D, int NT, bool SPLIT8 = false, bool PERM = false>
__device__ __forceinline__ void stage_rows_raw(const ChunkRegs<TIn, D, NT>& cr, int tid,
                                               typename Mma<TIn>::op_t* rm, int ld) {
    static_assert(!PERM || sizeof(TIn) == 2, "the permuted layout is for bf16 rows");
#pragma unroll
    for (int j = 0; j < ChunkRegs<TIn, D, NT>::NV; ++j) {
        const int row = ChunkRegs<TIn, D, NT>::row_of(j, tid);
        const int col = ChunkRegs<TIn, D, NT>::col_of(j, tid);
        if constexpr (PERM) {
            *reinterpret_cast<uint2*>(rm + row * ld + pcol(col)) = make_uint2(cr.r[j].x, cr.r[j].y);
            *reinterpret_cast<uint2*>(rm + row * ld + pcol(col + 4)) = make_uint2(cr.r[j].z, cr.r[j].w);
        } else if constexpr (SPLIT8) {
            uint2* d = reinterpret_cast<uint2*>(rm + row * ld + col);
            d[0] = make_uint2(cr.r[j].x, cr.r[j].y);
            d[1] = make_uint2(cr.r[j].z, cr.r[j].w);
        } else {
            *reinterpret_cast<uint4*>(rm + row * ld + col) = cr.r[j];
        }
    }
}

}  // namespace la
