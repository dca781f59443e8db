// Internal helpers shared by the gfx950 kernels of the ternary linear layer.
//
// Code format ([trdm] trdm.cn "三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战"
// §3.1; [nxbn] m.nxbn.cn/news/169761 §2.2): 2 bits per weight, 00 -> 0,
// 01 -> +1, 10 -> -1, 11 -> 0; four codes per byte, the first weight in the
// lowest two bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ternary {

// Cache policy of the code loads of the decode and few-token kernels, a
// template parameter of each kernel (the immediate of the buffer load):
// kStreamLoad, non-temporal (the `nt` bit of gfx950 buffer loads), for
// launches whose problems all hold tiled codes, where every code byte is read
// once: the code stream then passes through the caches without displacing
// lines that are reused (x, scales).  On MI355X it took the fused 7B-shaped
// decode layer at one token from 14.2 to 12.9 us.  Row-major codes keep the
// default policy (0): consecutive slabs read the two halves of a row's
// 128-byte line, and a non-temporal first half loses the line before the
// second (the same layer slowed by 7 %).  Group scales keep it too (one line
// of a row's scales serves many slabs), and so does the prefill GEMM, which
// reads each weight tile once per token tile.  The policy is chosen per launch
// on the host rather than by a branch in the kernel: a branch between two
// load variants made the compiler's wait counts coarser (full drains instead
// of per-load waits) and cost more than the policy gained.
constexpr int kStreamLoad = 2;

template <int CP>
__device__ __forceinline__ auto load_codes(__amdgpu_buffer_rsrc_t rsrc, int off)
{
    static_assert(CP == 0 || CP == kStreamLoad, "code-load policy");
    return __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, CP);
}

// N such loads, w[j] from byte offset off(j), issued in order (a scheduling
// fence after each).
template <int CP, int N, class V, class Off>
__device__ __forceinline__ void load_code_run(V (&w)[N], __amdgpu_buffer_rsrc_t rsrc, Off off)
{
#pragma unroll
    for (int j = 0; j < N; ++j) {
        w[j] = load_codes<CP>(rsrc, off(j));
        __builtin_amdgcn_sched_barrier(0);
    }
}

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

// ---------------------------------------------------------------- rounding

// fp32 -> bf16 bit pattern: gfx950's conversion instruction (v_cvt_pk_bf16_f32),
// round to nearest even under the default rounding mode; NaN stays a NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// fp32 -> IEEE binary16 bit pattern (hardware conversion, round to nearest even).
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f)
{
    _Float16 h = (_Float16)f;
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b)
{
    return (float)__builtin_bit_cast(_Float16, b);
}

template <bool FP16>
__device__ __forceinline__ uint16_t round_out(float f)
{
    return FP16 ? f32_to_f16_rne(f) : f32_to_bf16_rne(f);
}

// ---------------------------------------------------------------- decode
//
// Sixteen 2-bit codes in one 32-bit word (code i in bits [2i+1:2i]) become
// eight 32-bit words, each holding two 16-bit weights in natural k order:
//   out[2j]   = {weight 4j,   weight 4j+1}    (low half, high half)
//   out[2j+1] = {weight 4j+2, weight 4j+3}
// Each 16-bit weight is +2.0 (0x4000), -2.0 (0xC000), +0 or -0 (code 11).
// These bit patterns mean +-2 in both bf16 and fp16, so callers fold the
// factor 1/2 into the scale.  No branches, no table: 17 VALU ops per word.
//
// Step 1 rewrites every field (b1 b0) as (sign, magnitude) = (b1, b0 ^ b1):
//   00 -> 00, 01 -> 01, 10 -> 11, 11 -> 10.
// Step 2 isolates field p of every byte at that byte's top two bits.
// Step 3 byte-permutes those tops into the high byte of each 16-bit half
// (v_perm_b32; selector 0x0c yields a zero byte).
__device__ __forceinline__ void decode16(uint32_t w, uint32_t out[8])
{
    // (sign, magnitude): even bits w ^ (w >> 1) = b0 ^ b1, odd bits w = b1, as
    // one three-input bit operation (truth table 0x78 of (w, w >> 1, mask):
    // mask ? w ^ (w >> 1) : w).
    const uint32_t z = __builtin_amdgcn_bitop3_b32(w, w >> 1, 0x55555555u, 0x78);
    const uint32_t z3 = z & 0xc0c0c0c0u;                               // field 3 of each byte
    const uint32_t z2 = (z << 2) & 0xc0c0c0c0u;                        // field 2
    const uint32_t z1 = (z << 4) & 0xc0c0c0c0u;                        // field 1
    const uint32_t z0 = (z << 6) & 0xc0c0c0c0u;                        // field 0
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // D.byte1 = S1.byte j, D.byte3 = S0.byte j, D.byte0 = D.byte2 = 0.
        const uint32_t sel = 0x000c000cu | (uint32_t)j << 8 | (uint32_t)(4 + j) << 24;
        out[2 * j] = __builtin_amdgcn_perm(z1, z0, sel);
        out[2 * j + 1] = __builtin_amdgcn_perm(z3, z2, sel);
    }
}

// Code 2-bit field -> int8 value, four codes of a byte-spread word at once:
// every byte of `spread` holds one code in its low two bits.
__device__ __forceinline__ uint32_t codes_to_i8x4(uint32_t spread)
{
    // LUT bytes: code 0 -> 0x00, 1 -> 0x01, 2 -> 0xff, 3 -> 0x00.
    return __builtin_amdgcn_perm(0u, 0x00ff0100u, spread);
}

}  // namespace ternary
