// common.h -- device helpers shared by the gfx950 kernels of this library.
//
// MFMA fragment conventions (CDNA4 wave64, 16x16 output tiles):
//   * output / accumulator D (16x16, f32x4 per lane): lane l holds
//     D[4*(l/16) + r][l%16], r = 0..3.
//   * an operand fragment covers one K-block: 32 k-values for bf16
//     (v_mfma_f32_16x16x32_bf16, 8 values per lane) and 16 k-values for fp32
//     (four v_mfma_f32_16x16x4_f32, 4 values per lane, value s used by the
//     s-th instruction).  Lane l supplies row/column l%16 of its operand and
//     a lane-group g = l/16 slice of the K-block.  Because the instruction
//     sums over k, any assignment of k-values to (g, slot) works as long as A
//     and B use the same one.  Two assignments are used:
//       contig : group g holds k = kb0 + (KB/4)*g + s          (one 16-byte LDS read)
//       accperm: group g holds k = kb0 + 4g + s  (s<4) and kb0 + 16 + 4g + (s-4)
//                which is exactly what a pair of accumulator tiles
//                stacked along k holds per lane; for fp32 the two coincide.
//     accperm lets a fp32 accumulator (e.g. the fast-weight state) feed the
//     next contraction straight from registers, with no LDS round trip.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define TTT_DEV __device__ __forceinline__

TTT_DEV float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
// round-to-nearest-even fp32 -> bf16 (hardware conversion on gfx950)
TTT_DEV uint16_t f2bf(float x) { return __builtin_bit_cast(uint16_t, (bf16_t)x); }
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// two floats -> packed bf16 pair (one v_cvt_pk_bf16_f32, round to nearest even)
TTT_DEV uint32_t pack2bf(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

TTT_DEV f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// The dispatcher hands workgroups to the 8 XCDs round-robin in linear
// workgroup order (XCD = id % 8), and each XCD has its own L2.  This maps the
// hardware id to a logical id such that every XCD runs one contiguous range
// of logical ids; ordering tiles by logical id then keeps tiles that share
// operands on one L2.  A bijection on [0, n).
TTT_DEV int xcd_logical(int id, int n) {
    const int q = n >> 3, r = n & 7, x = id & 7, k = id >> 3;
    return (x < r) ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

// One step of a direct-to-LDS load ring: issue(wa, wb) starts the loads
// that fill a later step's buffers, compute(ra, rb) reads this step's.  The
// ring orders its loads before the reads itself (s_waitcnt vmcnt on the
// wave's own loads, then a barrier).  The compiler, which cannot follow that,
// makes an LDS read wait for every LDS-bound load still in flight unless it
// can prove the two apart; it can when the written and the read buffers
// reach it as distinct __restrict__ parameters of one inlined call.  Without
// that proof every step would drain the whole ring before its first read.
// The buffers of a ring belong to one __shared__ array: the compiler tags
// every access to an LDS array with that array, and tagged loads and reads
// of one array look alike to it again.  The loads are issued before
// anything of the computation (the scheduler would otherwise sink them).
typedef __attribute__((address_space(3))) void lds_void_t;
template <class Issue, class Compute>
TTT_DEV void ring_step1(bf16_t* __restrict__ w, const bf16_t* __restrict__ r, Issue&& issue, Compute&& compute) {
    issue(w);
    __builtin_amdgcn_sched_barrier(0);
    compute(r);
}
template <class Issue, class Compute>
TTT_DEV void ring_step(bf16_t* __restrict__ wa, bf16_t* __restrict__ wb, const bf16_t* __restrict__ ra,
                       const bf16_t* __restrict__ rb, Issue&& issue, Compute&& compute) {
    issue(wa, wb);
    __builtin_amdgcn_sched_barrier(0);
    compute(ra, rb);
}

// ---------------------------------------------------------------- type traits
template <typename T> struct Tr;

template <> struct Tr<float> {
    static constexpr int KB = 16;           // k-values per operand fragment
    using frag = f32x4;                     // 16 bytes per lane
    static constexpr int ESZ = 4;
};
template <> struct Tr<bf16_t> {
    static constexpr int KB = 32;
    using frag = bf16x8;
    static constexpr int ESZ = 2;
};

// one K-block of D += A*B (A, B fragments in the same k-assignment)
TTT_DEV void mma(f32x4& acc, const f32x4& a, const f32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
}
TTT_DEV void mma(f32x4& acc, const bf16x8& a, const bf16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

// ------------------------------------------------------------ LDS fragments
// `row` points at element 0 of the lane's row; kb0 = first k of the block.
template <typename T>
TTT_DEV typename Tr<T>::frag ld_contig(const T* row, int kb0, int g) {
    return *reinterpret_cast<const typename Tr<T>::frag*>(row + kb0 + (Tr<T>::KB / 4) * g);
}
TTT_DEV f32x4 ld_accperm(const float* row, int kb0, int g) {
    return *reinterpret_cast<const f32x4*>(row + kb0 + 4 * g);
}
TTT_DEV bf16x8 ld_accperm(const bf16_t* row, int kb0, int g) {
    const u32x2 lo = *reinterpret_cast<const u32x2*>(row + kb0 + 4 * g);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(row + kb0 + 16 + 4 * g);
    const u32x4 w = u32x4{lo[0], lo[1], hi[0], hi[1]};
    return __builtin_bit_cast(bf16x8, w);
}

// accumulator tiles -> operand fragment in the accperm assignment
TTT_DEV f32x4 acc_to_frag(const f32x4& t0, const f32x4& /*unused*/, float*) { return t0; }
TTT_DEV bf16x8 acc_to_frag_bf16(const f32x4& t0, const f32x4& t1) {
    const u32x4 w = u32x4{pack2bf(t0[0], t0[1]), pack2bf(t0[2], t0[3]),
                          pack2bf(t1[0], t1[1]), pack2bf(t1[2], t1[3])};
    return __builtin_bit_cast(bf16x8, w);
}

// store 4 consecutive values (one accumulator tile column slice) to memory
TTT_DEV void st4(float* p, const f32x4& v) { *reinterpret_cast<f32x4*>(p) = v; }
TTT_DEV void st4(bf16_t* p, const f32x4& v) {
    *reinterpret_cast<u32x2*>(p) = u32x2{pack2bf(v[0], v[1]), pack2bf(v[2], v[3])};
}
