// Issue-rate probes: the vector-ALU ceiling the pair kernels are measured
// against, taken on the device itself instead of derived from a data sheet.
//
// Each probe kernel runs a fixed instruction sequence written in inline
// assembly (so the count per iteration is exact) over many iterations, with
// four independent chains interleaved so that no instruction waits on the one
// before it; the grid fills every SIMD with 8 waves. The pair probes repeat
// the instruction mix of one point pair of the d = 3 dense half-step:
//   fp32 (the shipped loop): 3 v_sub_f32 (row coordinate minus a scalar
//        column coordinate), v_fma_f32 + 2 v_fmac_f32 (squared distance, the
//        row shift folded into the first), v_fma_f32 (exponent with the
//        scalar column term), v_exp_f32, v_add_f32 (sum): 8 VALU + 1 exp;
//   fp64: 3 v_add_f64, 3 v_fma_f64, v_fma_f64, v_cvt_f32_f64, v_exp_f32,
//        v_add_f32: 9 VALU + 1 exp;
//   tile-local expanded form (the column's offset from its block origin
//        and its weight in SGPRs): v_mul_f32 + 2 v_fmac_f32 (the row's
//        scaled offset dotted with the column's), v_exp_f32, v_fmac_f32
//        (weighted sum): 4 VALU + 1 exp;
//   split form (the precise dense default): 3 v_sub_f32, v_mul_f32 +
//        2 v_fmac_f32 (squared distance), v_sub_f32 (integer column term
//        minus the row's integer shift), v_fmac_f32 (exponent), v_exp_f32,
//        v_fmac_f32 (weighted sum): 9 VALU + 1 exp.
// No result is meaningful; the probes only take time. A transcendental's
// result is read no earlier than three instructions after it is written.
#include "internal.h"

namespace sk {
namespace {

constexpr int kProbeThreads = 256;

// 4 independent fp32 FMA chains (VOP3, VGPR operands only).
__device__ __forceinline__ void body_fma_f32(float (&a)[4], float b, float c) {
  asm volatile(
      "v_fma_f32 %0, %4, %5, %0\n"
      "v_fma_f32 %1, %4, %5, %1\n"
      "v_fma_f32 %2, %4, %5, %2\n"
      "v_fma_f32 %3, %4, %5, %3\n"
      : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3])
      : "v"(b), "v"(c));
}

// 4 independent v_exp_f32 (each reads the previous one's result of its own
// chain four instructions later).
__device__ __forceinline__ void body_exp(float (&a)[4]) {
  asm volatile(
      "v_exp_f32 %0, %0\n"
      "v_exp_f32 %1, %1\n"
      "v_exp_f32 %2, %2\n"
      "v_exp_f32 %3, %3\n"
      : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
}

// 4 independent fp64 FMA chains.
__device__ __forceinline__ void body_fma_f64(double (&a)[4], double b, double c) {
  asm volatile(
      "v_fma_f64 %0, %4, %5, %0\n"
      "v_fma_f64 %1, %4, %5, %1\n"
      "v_fma_f64 %2, %4, %5, %2\n"
      "v_fma_f64 %3, %4, %5, %3\n"
      : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3])
      : "v"(b), "v"(c));
}

// 4 independent chains of v_sub_f32 with a scalar first operand (VOP2).
__device__ __forceinline__ void body_sub_sgpr(float (&a)[4], float s) {
  asm volatile(
      "v_sub_f32 %0, %4, %0\n"
      "v_sub_f32 %1, %4, %1\n"
      "v_sub_f32 %2, %4, %2\n"
      "v_sub_f32 %3, %4, %3\n"
      : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3])
      : "s"(s));
}

// 4 independent chains of v_fmac_f32 (VOP2, accumulator in the destination).
__device__ __forceinline__ void body_fmac(float (&a)[4], float b) {
  asm volatile(
      "v_fmac_f32 %0, %4, %4\n"
      "v_fmac_f32 %1, %4, %4\n"
      "v_fmac_f32 %2, %4, %4\n"
      "v_fmac_f32 %3, %4, %4\n"
      : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3])
      : "v"(b));
}

// 4 independent chains of v_add_f64 with a scalar operand.
__device__ __forceinline__ void body_add_f64(double (&a)[4], double s) {
  asm volatile(
      "v_add_f64 %0, %4, %0\n"
      "v_add_f64 %1, %4, %1\n"
      "v_add_f64 %2, %4, %2\n"
      "v_add_f64 %3, %4, %3\n"
      : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3])
      : "s"(s));
}

// 4 independent v_cvt_f32_f64 (fp64 sources, fp32 results).
__device__ __forceinline__ void body_cvt(const double (&a)[4], float (&r)[4]) {
  asm volatile(
      "v_cvt_f32_f64 %0, %4\n"
      "v_cvt_f32_f64 %1, %5\n"
      "v_cvt_f32_f64 %2, %6\n"
      "v_cvt_f32_f64 %3, %7\n"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
}

// One pair of the fp32 shifted loop for each of 4 rows against one column
// (y0, y1, y2, h in SGPRs); with_exp = false replaces the exp2 by nothing
// (the sum then adds the exponent itself).
template <bool with_exp>
__device__ __forceinline__ void body_pair_f32(const float (&x)[4][3], const float (&u)[4],
                                              float (&acc)[4], float nk, float y0, float y1,
                                              float y2, float h) {
  float d0[4], d1[4], d2[4], q[4], z[4];
  asm volatile(
      "v_sub_f32 %[a0], %[y0], %[x00]\n"
      "v_sub_f32 %[a1], %[y0], %[x10]\n"
      "v_sub_f32 %[a2], %[y0], %[x20]\n"
      "v_sub_f32 %[a3], %[y0], %[x30]\n"
      "v_sub_f32 %[b0], %[y1], %[x01]\n"
      "v_sub_f32 %[b1], %[y1], %[x11]\n"
      "v_sub_f32 %[b2], %[y1], %[x21]\n"
      "v_sub_f32 %[b3], %[y1], %[x31]\n"
      "v_sub_f32 %[c0], %[y2], %[x02]\n"
      "v_sub_f32 %[c1], %[y2], %[x12]\n"
      "v_sub_f32 %[c2], %[y2], %[x22]\n"
      "v_sub_f32 %[c3], %[y2], %[x32]\n"
      "v_fma_f32 %[q0], %[a0], %[a0], %[u0]\n"
      "v_fma_f32 %[q1], %[a1], %[a1], %[u1]\n"
      "v_fma_f32 %[q2], %[a2], %[a2], %[u2]\n"
      "v_fma_f32 %[q3], %[a3], %[a3], %[u3]\n"
      "v_fmac_f32 %[q0], %[b0], %[b0]\n"
      "v_fmac_f32 %[q1], %[b1], %[b1]\n"
      "v_fmac_f32 %[q2], %[b2], %[b2]\n"
      "v_fmac_f32 %[q3], %[b3], %[b3]\n"
      "v_fmac_f32 %[q0], %[c0], %[c0]\n"
      "v_fmac_f32 %[q1], %[c1], %[c1]\n"
      "v_fmac_f32 %[q2], %[c2], %[c2]\n"
      "v_fmac_f32 %[q3], %[c3], %[c3]\n"
      "v_fma_f32 %[z0], %[q0], %[nk], %[h]\n"
      "v_fma_f32 %[z1], %[q1], %[nk], %[h]\n"
      "v_fma_f32 %[z2], %[q2], %[nk], %[h]\n"
      "v_fma_f32 %[z3], %[q3], %[nk], %[h]\n"
      : [a0] "=&v"(d0[0]), [a1] "=&v"(d0[1]), [a2] "=&v"(d0[2]), [a3] "=&v"(d0[3]),
        [b0] "=&v"(d1[0]), [b1] "=&v"(d1[1]), [b2] "=&v"(d1[2]), [b3] "=&v"(d1[3]),
        [c0] "=&v"(d2[0]), [c1] "=&v"(d2[1]), [c2] "=&v"(d2[2]), [c3] "=&v"(d2[3]),
        [q0] "=&v"(q[0]), [q1] "=&v"(q[1]), [q2] "=&v"(q[2]), [q3] "=&v"(q[3]),
        [z0] "=&v"(z[0]), [z1] "=&v"(z[1]), [z2] "=&v"(z[2]), [z3] "=&v"(z[3])
      : [x00] "v"(x[0][0]), [x01] "v"(x[0][1]), [x02] "v"(x[0][2]), [x10] "v"(x[1][0]),
        [x11] "v"(x[1][1]), [x12] "v"(x[1][2]), [x20] "v"(x[2][0]), [x21] "v"(x[2][1]),
        [x22] "v"(x[2][2]), [x30] "v"(x[3][0]), [x31] "v"(x[3][1]), [x32] "v"(x[3][2]),
        [u0] "v"(u[0]), [u1] "v"(u[1]), [u2] "v"(u[2]), [u3] "v"(u[3]), [nk] "v"(nk),
        [y0] "s"(y0), [y1] "s"(y1), [y2] "s"(y2), [h] "s"(h));
  if (with_exp) {
    asm volatile(
        "v_exp_f32 %[z0], %[z0]\n"
        "v_exp_f32 %[z1], %[z1]\n"
        "v_exp_f32 %[z2], %[z2]\n"
        "v_exp_f32 %[z3], %[z3]\n"
        "v_add_f32 %[s0], %[s0], %[z0]\n"
        "v_add_f32 %[s1], %[s1], %[z1]\n"
        "v_add_f32 %[s2], %[s2], %[z2]\n"
        "v_add_f32 %[s3], %[s3], %[z3]\n"
        : [s0] "+v"(acc[0]), [s1] "+v"(acc[1]), [s2] "+v"(acc[2]), [s3] "+v"(acc[3]),
          [z0] "+v"(z[0]), [z1] "+v"(z[1]), [z2] "+v"(z[2]), [z3] "+v"(z[3]));
  } else {
    asm volatile(
        "v_add_f32 %[s0], %[s0], %[z0]\n"
        "v_add_f32 %[s1], %[s1], %[z1]\n"
        "v_add_f32 %[s2], %[s2], %[z2]\n"
        "v_add_f32 %[s3], %[s3], %[z3]\n"
        : [s0] "+v"(acc[0]), [s1] "+v"(acc[1]), [s2] "+v"(acc[2]), [s3] "+v"(acc[3])
        : [z0] "v"(z[0]), [z1] "v"(z[1]), [z2] "v"(z[2]), [z3] "v"(z[3]));
  }
}

// The same pair in fp64 up to the exponent, which is rounded to fp32 for the
// exp2: 3 v_add_f64 (row coordinate plus the negated scalar column
// coordinate, a kernel argument), v_fma_f64 + 2 v_fma_f64, v_fma_f64 (exponent with the scalar
// column term), v_cvt_f32_f64, v_exp_f32, v_add_f32, for 2 rows (the fp64
// registers of 4 rows would not leave room for 8 waves).
__device__ __forceinline__ void body_pair_f64(const double (&x)[2][3], const double (&u)[2],
                                              float (&acc)[2], double nk, double y0, double y1,
                                              double y2, double h) {
  double d0[2], d1[2], d2[2], q[2];
  float z[2];
  asm volatile(
      "v_add_f64 %[a0], %[y0], %[x00]\n"
      "v_add_f64 %[a1], %[y0], %[x10]\n"
      "v_add_f64 %[b0], %[y1], %[x01]\n"
      "v_add_f64 %[b1], %[y1], %[x11]\n"
      "v_add_f64 %[c0], %[y2], %[x02]\n"
      "v_add_f64 %[c1], %[y2], %[x12]\n"
      "v_fma_f64 %[q0], %[a0], %[a0], %[u0]\n"
      "v_fma_f64 %[q1], %[a1], %[a1], %[u1]\n"
      "v_fma_f64 %[q0], %[b0], %[b0], %[q0]\n"
      "v_fma_f64 %[q1], %[b1], %[b1], %[q1]\n"
      "v_fma_f64 %[q0], %[c0], %[c0], %[q0]\n"
      "v_fma_f64 %[q1], %[c1], %[c1], %[q1]\n"
      "v_fma_f64 %[q0], %[q0], %[nk], %[h]\n"
      "v_fma_f64 %[q1], %[q1], %[nk], %[h]\n"
      "v_cvt_f32_f64 %[z0], %[q0]\n"
      "v_cvt_f32_f64 %[z1], %[q1]\n"
      "v_exp_f32 %[z0], %[z0]\n"
      "v_exp_f32 %[z1], %[z1]\n"
      "s_nop 1\n"
      "v_add_f32 %[s0], %[s0], %[z0]\n"
      "v_add_f32 %[s1], %[s1], %[z1]\n"
      : [a0] "=&v"(d0[0]), [a1] "=&v"(d0[1]), [b0] "=&v"(d1[0]), [b1] "=&v"(d1[1]),
        [c0] "=&v"(d2[0]), [c1] "=&v"(d2[1]), [q0] "=&v"(q[0]), [q1] "=&v"(q[1]),
        [z0] "=&v"(z[0]), [z1] "=&v"(z[1]), [s0] "+v"(acc[0]), [s1] "+v"(acc[1])
      : [x00] "v"(x[0][0]), [x01] "v"(x[0][1]), [x02] "v"(x[0][2]), [x10] "v"(x[1][0]),
        [x11] "v"(x[1][1]), [x12] "v"(x[1][2]), [u0] "v"(u[0]), [u1] "v"(u[1]), [nk] "v"(nk),
        [y0] "s"(y0), [y1] "s"(y1), [y2] "s"(y2), [h] "s"(h));
}

// One pair of the tile-local expanded form for each of 4 rows against one
// column: p = a2 dy2 + a1 dy1 + a0 dy0 (the row's scaled offsets a in
// VGPRs, the column's offsets dy in SGPRs), T += w exp2(p) (w in an SGPR).
__device__ __forceinline__ void body_pair_tile(const float (&a)[4][3], float (&acc)[4], float dy0,
                                               float dy1, float dy2, float w) {
  float p[4];
  asm volatile(
      "v_mul_f32 %[p0], %[y2], %[a02]\n"
      "v_mul_f32 %[p1], %[y2], %[a12]\n"
      "v_mul_f32 %[p2], %[y2], %[a22]\n"
      "v_mul_f32 %[p3], %[y2], %[a32]\n"
      "v_fmac_f32 %[p0], %[y1], %[a01]\n"
      "v_fmac_f32 %[p1], %[y1], %[a11]\n"
      "v_fmac_f32 %[p2], %[y1], %[a21]\n"
      "v_fmac_f32 %[p3], %[y1], %[a31]\n"
      "v_fmac_f32 %[p0], %[y0], %[a00]\n"
      "v_fmac_f32 %[p1], %[y0], %[a10]\n"
      "v_fmac_f32 %[p2], %[y0], %[a20]\n"
      "v_fmac_f32 %[p3], %[y0], %[a30]\n"
      "v_exp_f32 %[p0], %[p0]\n"
      "v_exp_f32 %[p1], %[p1]\n"
      "v_exp_f32 %[p2], %[p2]\n"
      "v_exp_f32 %[p3], %[p3]\n"
      "v_fmac_f32 %[s0], %[w], %[p0]\n"
      "v_fmac_f32 %[s1], %[w], %[p1]\n"
      "v_fmac_f32 %[s2], %[w], %[p2]\n"
      "v_fmac_f32 %[s3], %[w], %[p3]\n"
      : [p0] "=&v"(p[0]), [p1] "=&v"(p[1]), [p2] "=&v"(p[2]), [p3] "=&v"(p[3]),
        [s0] "+v"(acc[0]), [s1] "+v"(acc[1]), [s2] "+v"(acc[2]), [s3] "+v"(acc[3])
      : [a00] "v"(a[0][0]), [a01] "v"(a[0][1]), [a02] "v"(a[0][2]), [a10] "v"(a[1][0]),
        [a11] "v"(a[1][1]), [a12] "v"(a[1][2]), [a20] "v"(a[2][0]), [a21] "v"(a[2][1]),
        [a22] "v"(a[2][2]), [a30] "v"(a[3][0]), [a31] "v"(a[3][1]), [a32] "v"(a[3][2]),
        [y0] "s"(dy0), [y1] "s"(dy1), [y2] "s"(dy2), [w] "s"(w));
}

// One pair of the split form for each of 4 rows against one column (y0, y1,
// y2, the integer column term h and the weight w in SGPRs; the rows' integer
// shifts c and -kappa in VGPRs).
__device__ __forceinline__ void body_pair_split(const float (&x)[4][3], const float (&c)[4],
                                                float (&acc)[4], float nk, float y0, float y1,
                                                float y2, float h, float w) {
  float q[4], t[4];
  asm volatile(
      "v_sub_f32 %[q0], %[y0], %[x00]\n"
      "v_sub_f32 %[q1], %[y0], %[x10]\n"
      "v_sub_f32 %[q2], %[y0], %[x20]\n"
      "v_sub_f32 %[q3], %[y0], %[x30]\n"
      "v_mul_f32 %[q0], %[q0], %[q0]\n"
      "v_mul_f32 %[q1], %[q1], %[q1]\n"
      "v_mul_f32 %[q2], %[q2], %[q2]\n"
      "v_mul_f32 %[q3], %[q3], %[q3]\n"
      "v_sub_f32 %[t0], %[y1], %[x01]\n"
      "v_sub_f32 %[t1], %[y1], %[x11]\n"
      "v_sub_f32 %[t2], %[y1], %[x21]\n"
      "v_sub_f32 %[t3], %[y1], %[x31]\n"
      "v_fmac_f32 %[q0], %[t0], %[t0]\n"
      "v_fmac_f32 %[q1], %[t1], %[t1]\n"
      "v_fmac_f32 %[q2], %[t2], %[t2]\n"
      "v_fmac_f32 %[q3], %[t3], %[t3]\n"
      "v_sub_f32 %[t0], %[y2], %[x02]\n"
      "v_sub_f32 %[t1], %[y2], %[x12]\n"
      "v_sub_f32 %[t2], %[y2], %[x22]\n"
      "v_sub_f32 %[t3], %[y2], %[x32]\n"
      "v_fmac_f32 %[q0], %[t0], %[t0]\n"
      "v_fmac_f32 %[q1], %[t1], %[t1]\n"
      "v_fmac_f32 %[q2], %[t2], %[t2]\n"
      "v_fmac_f32 %[q3], %[t3], %[t3]\n"
      "v_sub_f32 %[t0], %[h], %[c0]\n"
      "v_sub_f32 %[t1], %[h], %[c1]\n"
      "v_sub_f32 %[t2], %[h], %[c2]\n"
      "v_sub_f32 %[t3], %[h], %[c3]\n"
      "v_fmac_f32 %[t0], %[q0], %[nk]\n"
      "v_fmac_f32 %[t1], %[q1], %[nk]\n"
      "v_fmac_f32 %[t2], %[q2], %[nk]\n"
      "v_fmac_f32 %[t3], %[q3], %[nk]\n"
      "v_exp_f32 %[t0], %[t0]\n"
      "v_exp_f32 %[t1], %[t1]\n"
      "v_exp_f32 %[t2], %[t2]\n"
      "v_exp_f32 %[t3], %[t3]\n"
      "v_fmac_f32 %[s0], %[w], %[t0]\n"
      "v_fmac_f32 %[s1], %[w], %[t1]\n"
      "v_fmac_f32 %[s2], %[w], %[t2]\n"
      "v_fmac_f32 %[s3], %[w], %[t3]\n"
      : [q0] "=&v"(q[0]), [q1] "=&v"(q[1]), [q2] "=&v"(q[2]), [q3] "=&v"(q[3]),
        [t0] "=&v"(t[0]), [t1] "=&v"(t[1]), [t2] "=&v"(t[2]), [t3] "=&v"(t[3]),
        [s0] "+v"(acc[0]), [s1] "+v"(acc[1]), [s2] "+v"(acc[2]), [s3] "+v"(acc[3])
      : [x00] "v"(x[0][0]), [x01] "v"(x[0][1]), [x02] "v"(x[0][2]), [x10] "v"(x[1][0]),
        [x11] "v"(x[1][1]), [x12] "v"(x[1][2]), [x20] "v"(x[2][0]), [x21] "v"(x[2][1]),
        [x22] "v"(x[2][2]), [x30] "v"(x[3][0]), [x31] "v"(x[3][1]), [x32] "v"(x[3][2]),
        [c0] "v"(c[0]), [c1] "v"(c[1]), [c2] "v"(c[2]), [c3] "v"(c[3]), [nk] "v"(nk),
        [y0] "s"(y0), [y1] "s"(y1), [y2] "s"(y2), [h] "s"(h), [w] "s"(w));
}

typedef float v4f __attribute__((ext_vector_type(4)));

// The tile-local expanded form with the cross terms on the matrix cores, as
// the sparse half-step runs it: four 16 x 16 pair blocks, each a chain of 3
// v_mfma_f32_4x4x1_16b_f32 (one per coordinate), then per lane 4 v_exp_f32
// and 4 v_fmac_f32 (the column weights) per block. The empty asm statements
// make the row operands opaque to the compiler each iteration, so the chains
// stay in the loop; they emit no instructions.
__device__ __forceinline__ void body_pair_tile_mfma(float (&b)[4][3], float (&acc)[4],
                                                    const float (&a)[3], const v4f& w) {
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) asm volatile("" : "+v"(b[rb][0]), "+v"(b[rb][1]), "+v"(b[rb][2]));
  v4f z[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
    z[rb] = __builtin_amdgcn_mfma_f32_4x4x1f32(a[0], b[rb][0], (v4f){0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
  for (int k = 1; k < 3; ++k)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) z[rb] = __builtin_amdgcn_mfma_f32_4x4x1f32(a[k], b[rb][k], z[rb], 0, 0, 0);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[rb] = __builtin_fmaf(w[v], __builtin_amdgcn_exp2f(z[rb][v]), acc[rb]);
}

template <int KIND>
__global__ __launch_bounds__(kProbeThreads) void k_probe(float* __restrict__ out, int32_t iters,
                                                        float s0, float s1, float s2, float s3,
                                                        double e0, double e1, double e2, double e3) {
  const float t = (float)threadIdx.x * 1e-6f;
  float acc[4] = {t, t + 1.0f, t + 2.0f, t + 3.0f};
  if constexpr (KIND == SINKHORN_PROBE_FMA_F32) {
    for (int32_t i = 0; i < iters; ++i) body_fma_f32(acc, s0, s1);
  } else if constexpr (KIND == SINKHORN_PROBE_EXP_F32) {
    for (int32_t i = 0; i < iters; ++i) body_exp(acc);
  } else if constexpr (KIND == SINKHORN_PROBE_FMA_F64) {
    double a[4] = {t, t + 1.0, t + 2.0, t + 3.0};
    for (int32_t i = 0; i < iters; ++i) body_fma_f64(a, (double)s0, (double)s1);
    acc[0] = (float)(a[0] + a[1] + a[2] + a[3]);
  } else if constexpr (KIND == SINKHORN_PROBE_SUB_F32) {
    for (int32_t i = 0; i < iters; ++i) body_sub_sgpr(acc, s0);
  } else if constexpr (KIND == SINKHORN_PROBE_FMAC_F32) {
    for (int32_t i = 0; i < iters; ++i) body_fmac(acc, s2);
  } else if constexpr (KIND == SINKHORN_PROBE_ADD_F64) {
    double a[4] = {t, t + 1.0, t + 2.0, t + 3.0};
    for (int32_t i = 0; i < iters; ++i) body_add_f64(a, e0);
    acc[0] = (float)(a[0] + a[1] + a[2] + a[3]);
  } else if constexpr (KIND == SINKHORN_PROBE_CVT_F32_F64) {
    const double a[4] = {t, t + 1.0, t + 2.0, t + 3.0};
    for (int32_t i = 0; i < iters; ++i) {
      float r[4];
      body_cvt(a, r);
      acc[0] += r[0] + r[1] + r[2] + r[3];
    }
  } else if constexpr (KIND == SINKHORN_PROBE_PAIR_F32 || KIND == SINKHORN_PROBE_PAIR_F32_NOEXP) {
    float x[4][3], u[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      u[r] = t * (float)(r + 1);
#pragma unroll
      for (int k = 0; k < 3; ++k) x[r][k] = t + 0.25f * (float)(r + k);
    }
    for (int32_t i = 0; i < iters; ++i)
      body_pair_f32<KIND == SINKHORN_PROBE_PAIR_F32>(x, u, acc, -1.0f, s0, s1, s2, s3);
  } else if constexpr (KIND == SINKHORN_PROBE_PAIR_TILE_F32) {
    float a[4][3];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int k = 0; k < 3; ++k) a[r][k] = t + 0.25f * (float)(r + k);
    for (int32_t i = 0; i < iters; ++i) body_pair_tile(a, acc, s0, s1, s2, s3);
  } else if constexpr (KIND == SINKHORN_PROBE_PAIR_TILE_MFMA) {
    float b[4][3];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int k = 0; k < 3; ++k) b[r][k] = 4.0f * t + 0.125f * (float)(r + k);
    const float a[3] = {0.5f * t, 0.25f - t, 0.125f + t};
    const v4f w = {0.5f, 0.25f, 0.125f, 0.0625f};
    for (int32_t i = 0; i < iters; ++i) body_pair_tile_mfma(b, acc, a, w);
  } else if constexpr (KIND == SINKHORN_PROBE_PAIR_SPLIT_F32) {
    float x[4][3], c[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      c[r] = (float)(r + 3);
#pragma unroll
      for (int k = 0; k < 3; ++k) x[r][k] = t + 0.25f * (float)(r + k);
    }
    for (int32_t i = 0; i < iters; ++i) body_pair_split(x, c, acc, -1.0f, s0, s1, s2, s3, 0.5f);
  } else if constexpr (KIND == SINKHORN_PROBE_PAIR_F64) {
    double x[2][3], u[2];
    float a2[2] = {acc[0], acc[1]};
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      u[r] = (double)t * (r + 1);
#pragma unroll
      for (int k = 0; k < 3; ++k) x[r][k] = (double)t + 0.25 * (r + k);
    }
    for (int32_t i = 0; i < iters; ++i)
      body_pair_f64(x, u, a2, -1.0, e0, e1, e2, e3);
    acc[0] = a2[0];
    acc[1] = a2[1];
  }
  out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc[0] + acc[1] + acc[2] + acc[3];
}

// Lane-instructions per iteration of the counted class (VALU without the
// transcendentals, or the transcendentals alone for the exp probe) and point
// pairs per iteration, per work-item.
void probe_counts(int32_t kind, double* valu, double* pairs) {
  switch (kind) {
    case SINKHORN_PROBE_FMA_F32: *valu = 4; *pairs = 0; break;
    case SINKHORN_PROBE_EXP_F32: *valu = 4; *pairs = 0; break;
    case SINKHORN_PROBE_FMA_F64: *valu = 4; *pairs = 0; break;
    case SINKHORN_PROBE_PAIR_F32: *valu = 32; *pairs = 4; break;
    case SINKHORN_PROBE_PAIR_F32_NOEXP: *valu = 32; *pairs = 4; break;
    case SINKHORN_PROBE_PAIR_F64: *valu = 18; *pairs = 2; break;
    case SINKHORN_PROBE_SUB_F32: *valu = 4; *pairs = 0; break;
    case SINKHORN_PROBE_FMAC_F32: *valu = 4; *pairs = 0; break;
    case SINKHORN_PROBE_ADD_F64: *valu = 4; *pairs = 0; break;
    case SINKHORN_PROBE_CVT_F32_F64: *valu = 4; *pairs = 0; break;
    case SINKHORN_PROBE_PAIR_TILE_F32: *valu = 16; *pairs = 4; break;
    case SINKHORN_PROBE_PAIR_SPLIT_F32: *valu = 36; *pairs = 4; break;
    // a wave's 4 blocks of 16 x 16 pairs: 16 pairs and 16 fmas per lane
    case SINKHORN_PROBE_PAIR_TILE_MFMA: *valu = 16; *pairs = 16; break;
    default: fail(SINKHORN_ERR_INVALID_ARG, "unknown probe kind");
  }
}

}  // namespace
}  // namespace sk

using namespace sk;

extern "C" int sinkhorn_probe_issue_rate(int32_t kind, int32_t iters, void* stream,
                                         double* lane_instr_per_s, double* pairs_per_s,
                                         double* kernel_ms) {
  try {
    if (iters < 1) fail(SINKHORN_ERR_INVALID_ARG, "iters must be >= 1");
    double valu = 0, pairs = 0;
    probe_counts(kind, &valu, &pairs);
    hipStream_t st = (hipStream_t)stream;
    int dev = 0, cus = 0;
    SK_HIP(hipGetDevice(&dev));
    SK_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    // 8 workgroups of 4 waves per CU: 8 waves on each of its 4 SIMDs
    const int64_t blocks = (int64_t)(cus > 0 ? cus : 1) * 8;
    float* out = (float*)dev_alloc(sizeof(float) * blocks * kProbeThreads);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    float ms = 0.0f;
    try {
      SK_HIP(hipEventCreate(&e0));
      SK_HIP(hipEventCreate(&e1));
      auto launch = [&](int32_t it) {
        switch (kind) {
#define SK_PROBE(K)                                                                           \
  case K:                                                                                     \
    hipLaunchKernelGGL(k_probe<K>, grid1(blocks, kProbeThreads), dim3(kProbeThreads), 0, st, \
                       out, it, 0.5f, 0.25f, 0.125f, -3.0f, -0.5, -0.25, -0.125, -3.0);       \
    break;
          SK_PROBE(SINKHORN_PROBE_FMA_F32)
          SK_PROBE(SINKHORN_PROBE_EXP_F32)
          SK_PROBE(SINKHORN_PROBE_FMA_F64)
          SK_PROBE(SINKHORN_PROBE_PAIR_F32)
          SK_PROBE(SINKHORN_PROBE_PAIR_F32_NOEXP)
          SK_PROBE(SINKHORN_PROBE_PAIR_F64)
          SK_PROBE(SINKHORN_PROBE_SUB_F32)
          SK_PROBE(SINKHORN_PROBE_FMAC_F32)
          SK_PROBE(SINKHORN_PROBE_ADD_F64)
          SK_PROBE(SINKHORN_PROBE_CVT_F32_F64)
          SK_PROBE(SINKHORN_PROBE_PAIR_TILE_F32)
          SK_PROBE(SINKHORN_PROBE_PAIR_SPLIT_F32)
          SK_PROBE(SINKHORN_PROBE_PAIR_TILE_MFMA)
#undef SK_PROBE
        }
        SK_LAUNCH_CHECK();
      };
      launch(1);  // warm-up: code object load, clocks
      SK_HIP(hipEventRecord(e0, st));
      launch(iters);
      SK_HIP(hipEventRecord(e1, st));
      SK_HIP(hipEventSynchronize(e1));
      SK_HIP(hipEventElapsedTime(&ms, e0, e1));
    } catch (...) {
      if (e0) (void)hipEventDestroy(e0);
      if (e1) (void)hipEventDestroy(e1);
      dev_free(out);
      throw;
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    dev_free(out);
    const double items = (double)blocks * kProbeThreads * (double)iters;
    const double sec = (double)ms * 1e-3;
    if (lane_instr_per_s) *lane_instr_per_s = sec > 0 ? items * valu / sec : 0.0;
    if (pairs_per_s) *pairs_per_s = sec > 0 ? items * pairs / sec : 0.0;
    if (kernel_ms) *kernel_ms = ms;
    return SINKHORN_OK;
  } catch (const Failure& e) {
    set_last_error(e.msg);
    return e.code;
  } catch (...) {
    set_last_error("unexpected exception");
    return SINKHORN_ERR_HIP;
  }
}
