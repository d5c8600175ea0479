// Block-scaled fp8 x fp4 matrix-instruction helpers shared by the decode and
// prefill kernels: fp8 limbs of activations in compact records, +-1 signs as
// fp4 operands, and the 16x16x128 instruction itself.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace lb {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

namespace {

constexpr int kRec = 144;                 // compact record: 128 fp8 bytes, 4 scales, padding

__device__ __forceinline__ float ldexp2(float v, int e) { return __builtin_amdgcn_ldexpf(v, e); }

// fp32 -> OCP e4m3 byte (round to nearest even; in range by construction)
__device__ __forceinline__ uint32_t to_fp8(float v) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xffu;
}
__device__ __forceinline__ float from_fp8(uint32_t b) {
    return __builtin_amdgcn_cvt_f32_fp8((int)b, 0);
}

// Where element e of a 128-element K-group goes.  The fp4 sign operand holds
// bit 4i+q of plane word g in MFMA slot s = 8q+i (fp4 lanes carry K = 32g+s);
// an fp8 operand holds K in lane group gp = (K mod 64)/16 at byte
// sp = (K mod 16) + 16*(K >= 64) (measured layout of the f8f6f4 instruction).
// In the LDS operand, activation row c of lane group gp is lane c + 16*gp
// (32 bytes); the scale of K-block g of row c sits in lane c + 16*g.
// In a compact record the row's four lane-group pieces follow each other.
__device__ __forceinline__ int rec_offset(int e) {
    const int g = e >> 5, bit = e & 31;
    const int s = ((bit & 3) << 3) | (bit >> 2);
    const int K = (g << 5) | s;
    const int gp = (K & 63) >> 4;
    const int sp = (K & 15) | ((K >> 6) << 4);
    return (gp << 5) + sp;
}

// The NL limbs of v into a compact record set: data points at (element, row
// c0) and row c0+q is kRec bytes further; scale points at the K-block scale of
// row c0; first = the lane holds element 0 of its 32-element block.  Called by
// whole waves: each 32-lane half handles one 32-element block, whose largest
// magnitude sets the scales 2^(E-7-4q).  Lanes with ok == false take part in
// the reduction with v = 0 and store nothing.
template <int NL>
__device__ __forceinline__ void emit_limbs(float v, uint8_t *data, uint8_t *scale, bool ok, bool first) {
    float m = fabsf(v);
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const int E = (int)((__float_as_uint(m) >> 23) & 0xff) - 127;   // floor(log2 m); m == 0 -> -127
    float r = v;
#pragma unroll
    for (int q = 0; q < NL; ++q) {
        const int eq = E - 7 - 4 * q;
        const uint32_t b = to_fp8(ldexp2(r, -eq));
        r -= ldexp2(from_fp8(b), eq);
        if (ok) {
            data[kRec * q] = (uint8_t)b;
            if (first) scale[kRec * q] = (uint8_t)(eq < -127 ? 0 : (eq > 127 ? 254 : eq + 127));
        }
    }
}

// (x & mask) | one with mask = 0x88888888 in an SGPR and one = 0x22222222 in
// a VGPR: a single v_and_or_b32 (VOP3 on gfx950 takes no literal operand, so
// the compiler would otherwise split it into an AND and an OR).
struct Nib {
    uint32_t mask, one;
};

__device__ __forceinline__ uint32_t sign_nibbles(uint32_t x, const Nib &k) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(k.mask), "v"(k.one));
    return r;
}

// The two constants of sign_nibbles in registers, opaque to constant folding.
__device__ __forceinline__ Nib nibble_constants() {
    Nib k;
    asm volatile("s_mov_b32 %0, 0x88888888" : "=s"(k.mask));
    asm volatile("v_mov_b32 %0, 0x22222222" : "=v"(k.one));
    return k;
}

// fp4 sign operand of one plane word: slot 8q+i <- bit 4i+q, as +-1.0.
__device__ __forceinline__ v8i unpack_word(uint32_t w, const Nib &k) {
    v8i a;
    a[0] = (int)sign_nibbles(w << 3, k);
    a[1] = (int)sign_nibbles(w << 2, k);
    a[2] = (int)sign_nibbles(w << 1, k);
    a[3] = (int)sign_nibbles(w, k);
    a[4] = a[5] = a[6] = a[7] = 0;
    return a;
}

// The fp4 sign operands of four plane words, two words per 64-bit shift: the
// bits a shift carries from the low word into the high one land at nibble bits
// 0..2, which the mask clears, so each word's operand is unpack_word's.  Three
// v_lshlrev_b64 replace six 32-bit shifts (written out: the compiler splits a
// 64-bit shift into a 32-bit shift and a v_alignbit_b32, two instructions).
__device__ __forceinline__ void unpack_quad(const v4u &w, const Nib &k, v8i sg[4]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint64_t W = ((uint64_t)w[2 * h + 1] << 32) | (uint64_t)w[2 * h];
        uint64_t W3, W2, W1;
        asm("v_lshlrev_b64 %0, 3, %1" : "=v"(W3) : "v"(W));
        asm("v_lshlrev_b64 %0, 2, %1" : "=v"(W2) : "v"(W));
        asm("v_lshlrev_b64 %0, 1, %1" : "=v"(W1) : "v"(W));
        v8i &lo = sg[2 * h], &hi = sg[2 * h + 1];
        lo[0] = (int)sign_nibbles((uint32_t)W3, k);
        lo[1] = (int)sign_nibbles((uint32_t)W2, k);
        lo[2] = (int)sign_nibbles((uint32_t)W1, k);
        lo[3] = (int)sign_nibbles((uint32_t)W, k);
        hi[0] = (int)sign_nibbles((uint32_t)(W3 >> 32), k);
        hi[1] = (int)sign_nibbles((uint32_t)(W2 >> 32), k);
        hi[2] = (int)sign_nibbles((uint32_t)(W1 >> 32), k);
        hi[3] = (int)sign_nibbles((uint32_t)(W >> 32), k);
        lo[4] = lo[5] = lo[6] = lo[7] = 0;
        hi[4] = hi[5] = hi[6] = hi[7] = 0;
    }
}

// 32 bytes at p (16-byte aligned) as an fp8 operand
__device__ __forceinline__ v8i load_op_at(const uint8_t *p) {
    const v4u lo = *(const v4u *)p, hi = *(const v4u *)(p + 16);
    v8i b;
    b[0] = (int)lo[0]; b[1] = (int)lo[1]; b[2] = (int)lo[2]; b[3] = (int)lo[3];
    b[4] = (int)hi[0]; b[5] = (int)hi[1]; b[6] = (int)hi[2]; b[7] = (int)hi[3];
    return b;
}

// acc += act (fp8, scale sa per lane) x signs (fp4, scale 1.0)
__device__ __forceinline__ v4f mfma_f8f4(const v8i &act, const v8i &sg, v4f c, int sa) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(act, sg, c, 0, 4, 0, sa, 0, 127);
}

}  // namespace
}  // namespace lb
