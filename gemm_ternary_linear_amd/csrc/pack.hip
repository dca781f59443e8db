// Pack / unpack of 2-bit ternary codes on gfx950, and the conversion between
// the row-major packing and the library's tiled layout.
//
// Format from [trdm] trdm.cn "三元量化模型接入vLLM：从逆向加载到Kernel优化的完整实战"
// §3.1 and [nxbn] m.nxbn.cn/news/169761 §2.2: value +1 -> code 01, -1 -> 10,
// 0 -> 00; code 11 is reserved and decodes to 0; four codes per byte, the
// first weight in the lowest two bits.
//
// Both buffers are contiguous and K % 4 == 0, so byte j of the packed buffer
// always holds values 4j..4j+3 of the flat int8 buffer, across row ends.  Each
// thread owns 16 packed bytes (64 values): one 16-byte access on the packed
// side, four on the int8 side.  These kernels are HBM-bound (5 bytes per 4
// weights); the arithmetic is a few VALU ops per byte.
#include "common.h"
#include "internal.h"

namespace ternary {

// One int8 value -> 2-bit code, plus whether it was outside {-1, 0, +1}.
__device__ __forceinline__ uint32_t encode_one(int8_t v, int &bad)
{
    bad += (v != 0) & (v != 1) & (v != -1);
    return (uint32_t)(v == 1) | ((uint32_t)(v == -1) << 1);
}

// Four values packed in the bytes of `d` (value i in byte i) -> one code byte.
__device__ __forceinline__ uint32_t encode4(uint32_t d, int &bad)
{
    uint32_t b = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        b |= encode_one((int8_t)(d >> (8 * i)), bad) << (2 * i);
    return b;
}

__global__ void __launch_bounds__(256) pack_kernel(const int8_t *__restrict__ q,
                                                   uint8_t *__restrict__ packed, int64_t nbytes,
                                                   int32_t *__restrict__ invalid_count)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t b0 = t * 16;
    int bad = 0;
    if (b0 + 16 <= nbytes) {
        const uint4 *src = reinterpret_cast<const uint4 *>(q + b0 * 4);
        uint32_t o[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const uint4 d = src[v];
            o[v] = encode4(d.x, bad) | encode4(d.y, bad) << 8 | encode4(d.z, bad) << 16 |
                   encode4(d.w, bad) << 24;
        }
        *reinterpret_cast<uint4 *>(packed + b0) = make_uint4(o[0], o[1], o[2], o[3]);
    } else if (b0 < nbytes) {
        for (int64_t b = b0; b < nbytes; ++b) {
            uint32_t d = (uint32_t)(uint8_t)q[4 * b] | (uint32_t)(uint8_t)q[4 * b + 1] << 8 |
                         (uint32_t)(uint8_t)q[4 * b + 2] << 16 |
                         (uint32_t)(uint8_t)q[4 * b + 3] << 24;
            packed[b] = (uint8_t)encode4(d, bad);
        }
    }
    if (invalid_count) {
        // Integer wave reduction, then one atomic per wave: the total is exact
        // whatever the order.
        for (int off = 32; off > 0; off >>= 1)
            bad += __shfl_xor(bad, off);
        if ((threadIdx.x & 63) == 0 && bad)
            atomicAdd(invalid_count, bad);
    }
}

// 16 codes of w -> four int8x4 words in natural order (values 4j..4j+3 in out[j]).
__device__ __forceinline__ void unpack_word(uint32_t w, uint32_t out[4])
{
    // s_p.byte j = code (4j + p), then a 4x4 byte transpose.
    const uint32_t t0 = codes_to_i8x4(w & 0x03030303u);
    const uint32_t t1 = codes_to_i8x4((w >> 2) & 0x03030303u);
    const uint32_t t2 = codes_to_i8x4((w >> 4) & 0x03030303u);
    const uint32_t t3 = codes_to_i8x4((w >> 6) & 0x03030303u);
    const uint32_t u0 = __builtin_amdgcn_perm(t1, t0, 0x05010400u);  // t0.b0 t1.b0 t0.b1 t1.b1
    const uint32_t u1 = __builtin_amdgcn_perm(t1, t0, 0x07030602u);  // t0.b2 t1.b2 t0.b3 t1.b3
    const uint32_t u2 = __builtin_amdgcn_perm(t3, t2, 0x05010400u);
    const uint32_t u3 = __builtin_amdgcn_perm(t3, t2, 0x07030602u);
    out[0] = __builtin_amdgcn_perm(u2, u0, 0x05040100u);            // t0.b0 t1.b0 t2.b0 t3.b0
    out[1] = __builtin_amdgcn_perm(u2, u0, 0x07060302u);
    out[2] = __builtin_amdgcn_perm(u3, u1, 0x05040100u);
    out[3] = __builtin_amdgcn_perm(u3, u1, 0x07060302u);
}

__global__ void __launch_bounds__(256) unpack_kernel(const uint8_t *__restrict__ packed,
                                                     int8_t *__restrict__ q, int64_t nbytes)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t b0 = t * 16;
    if (b0 + 16 <= nbytes) {
        const uint4 p = *reinterpret_cast<const uint4 *>(packed + b0);
        const uint32_t w[4] = {p.x, p.y, p.z, p.w};
        uint4 *dst = reinterpret_cast<uint4 *>(q + b0 * 4);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            uint32_t o[4];
            unpack_word(w[v], o);
            dst[v] = make_uint4(o[0], o[1], o[2], o[3]);
        }
    } else if (b0 < nbytes) {
        for (int64_t b = b0; b < nbytes; ++b) {
            const uint32_t byte = packed[b];
            const uint32_t v = codes_to_i8x4((byte & 3u) | ((byte >> 2) & 3u) << 8 |
                                             ((byte >> 4) & 3u) << 16 | (byte >> 6) << 24);
            for (int i = 0; i < 4; ++i)
                q[4 * b + i] = (int8_t)(v >> (8 * i));
        }
    }
}

// Tiled layout (the library's): 16-row x 256-code blocks of 1 KB, stored
// [4 quarters][16 rows][16 bytes] (quarter g = bytes 16g .. 16g+15 of the
// block's 64 bytes of each row), blocks of a row band consecutive.  Thread t
// owns tiled bytes 16t .. 16t+15: quarter g of row r of block (band, slab),
// i.e. row-major bytes j0 .. j0+15 of row n with
//   t = ((band * ks + slab) * 4 + g) * 16 + r,  n = 16 band + r,  j0 = 64 slab + 16 g.
// Bytes past N rows or K/4 columns are the zero padding.
struct TileUnit {
    int64_t n, j0;  // row and first row-major byte of the unit
};
__device__ __forceinline__ TileUnit tile_unit(int64_t t, int64_t ks)
{
    const int64_t r = t & 15, g = (t >> 4) & 3, blk = t >> 6;
    return {(blk / ks) * 16 + r, (blk % ks) * 64 + 16 * g};
}

__global__ void __launch_bounds__(256) tile_kernel(const uint8_t *__restrict__ packed, int64_t N,
                                                   int64_t K, uint8_t *__restrict__ tiled,
                                                   int64_t units)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= units)
        return;
    const int64_t rb = K >> 2, ks = (K + 255) >> 8;
    const TileUnit u = tile_unit(t, ks);
    uint32_t w[4] = {0, 0, 0, 0};
    if (u.n < N) {
        const uint8_t *src = packed + u.n * rb + u.j0;
        if ((rb & 15) == 0 && u.j0 + 16 <= rb) {
            const uint4 v = *reinterpret_cast<const uint4 *>(src);
            w[0] = v.x;
            w[1] = v.y;
            w[2] = v.z;
            w[3] = v.w;
        } else {
            for (int b = 0; b < 16; ++b)
                if (u.j0 + b < rb)
                    w[b >> 2] |= (uint32_t)src[b] << (8 * (b & 3));
        }
    }
    *reinterpret_cast<uint4 *>(tiled + 16 * t) = make_uint4(w[0], w[1], w[2], w[3]);
}

__global__ void __launch_bounds__(256) untile_kernel(const uint8_t *__restrict__ tiled, int64_t N,
                                                     int64_t K, uint8_t *__restrict__ packed,
                                                     int64_t units)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= units)
        return;
    const int64_t rb = K >> 2, ks = (K + 255) >> 8;
    const TileUnit u = tile_unit(t, ks);
    if (u.n >= N || u.j0 >= rb)
        return;
    const uint4 v = *reinterpret_cast<const uint4 *>(tiled + 16 * t);
    uint8_t *dst = packed + u.n * rb + u.j0;
    if ((rb & 15) == 0 && u.j0 + 16 <= rb) {
        *reinterpret_cast<uint4 *>(dst) = v;
    } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        for (int b = 0; b < 16; ++b)
            if (u.j0 + b < rb)
                dst[b] = (uint8_t)(w[b >> 2] >> (8 * (b & 3)));
    }
}

hipError_t launch_tile(const uint8_t *packed, int64_t N, int64_t K, uint8_t *tiled,
                       hipStream_t stream)
{
    const int64_t units = tiled_bytes(N, K) / 16;
    hipLaunchKernelGGL(tile_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, stream,
                       packed, N, K, tiled, units);
    return hipGetLastError();
}

hipError_t launch_untile(const uint8_t *tiled, int64_t N, int64_t K, uint8_t *packed,
                         hipStream_t stream)
{
    const int64_t units = tiled_bytes(N, K) / 16;
    hipLaunchKernelGGL(untile_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, stream,
                       tiled, N, K, packed, units);
    return hipGetLastError();
}

hipError_t launch_pack(const int8_t *q, int64_t nbytes, uint8_t *packed, int32_t *invalid_count,
                       hipStream_t stream)
{
    const int64_t threads = (nbytes + 15) / 16;
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, q, packed,
                       nbytes, invalid_count);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *packed, int64_t nbytes, int8_t *q, hipStream_t stream)
{
    const int64_t threads = (nbytes + 15) / 16;
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, packed, q,
                       nbytes);
    return hipGetLastError();
}

}  // namespace ternary
