// vq_device.h -- device-side building blocks shared by every VQ kernel:
// code extraction from packed words, codebook staging into LDS, and the
// codebook gather.  gfx950 (CDNA4), wave64.
//
// Format (paper "Data-Free Vector Quantization Beats Affine Quantization at
// Matched Bytes Below 5 Bits", §1 Notation and §2.3 Packing; model card
// "Qwen3.5-397B-A17B-VQ-2.4bpw", Methodology): code j of a row is the B bits
// starting at bit j*B of the row's little-endian code stream; rows hold whole
// 32-code blocks of B uint32 words.  Kernels work on "chunks" of 16
// consecutive codes of one row: 16*B bits, starting at byte 2*B*q of the row
// for chunk q.  For B = 8 and 12 that is 16 / 24 bytes from a 16- / 8-byte
// boundary.  Any other width is read as a window of whole words from the
// 4-byte boundary at or below the chunk (for odd B, odd chunks start 16 bits
// into a word) and shifted into place once the words have arrived.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vqmi {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCodesPerChunk = 16;

// ---------------------------------------------------------------------------
// buffer loads: one wave-uniform resource (base, size in bytes) in SGPRs and
// a 32-bit byte offset per lane.  Bytes at or past the size read as zero, so
// rows past the end of a tensor need no clamping.  Every buffer a kernel
// streams is below 2 GiB (the API checks).
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;  // an offset past every buffer

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0x7fffffffull ? 0x7fffffffu : (uint32_t)bytes;
  // dword 3 of a gfx9 buffer descriptor: 32-bit data format, raw addressing
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load_b128(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u32x2 buf_load_b64(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load_b32(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint16_t buf_load_b16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// codes
// ---------------------------------------------------------------------------

// Code widths with whole-word chunks on their natural boundaries.
template <int B>
constexpr bool kAlignedChunks = (B == 8 || B == 12);

// Words of one 16-code chunk: B / 2 for 8 and 12 bits; otherwise the
// (B + 1) / 2 words that cover 16*B bits from the 4-byte boundary at or below
// the chunk.
template <int B>
struct Chunk {
  static constexpr int kWords = kAlignedChunks<B> ? B / 2 : (B + 1) / 2;
  uint32_t w[kWords];
};

// Byte offset (4-byte aligned) of the words of chunk q within its row, and
// the bit offset of the chunk's first code in its first word (0 or 16).
template <int B>
__host__ __device__ constexpr uint32_t chunk_byte(uint32_t q) { return (2u * B * q) & ~3u; }
template <int B>
__device__ __forceinline__ uint32_t chunk_shift(uint32_t q) { return (B & 1) ? (q & 1u) * 16u : 0u; }

// N consecutive words from a 4-byte aligned byte offset (soffset: a
// wave-uniform part of the offset), in as few loads as the count allows.
template <int N>
__device__ __forceinline__ void load_words(uint32_t* w, rsrc_t r, uint32_t off, uint32_t soff = 0) {
  int k = 0;
#pragma unroll
  for (; k + 4 <= N; k += 4) {
    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 4u * k, soff, 0));
    w[k] = v.x; w[k + 1] = v.y; w[k + 2] = v.z; w[k + 3] = v.w;
  }
  if constexpr (N % 4 == 3) {
    typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
    const u32x3 v = __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(r, off + 4u * k, soff, 0));
    w[k] = v.x; w[k + 1] = v.y; w[k + 2] = v.z;
  } else if constexpr (N % 4 == 2) {
    const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off + 4u * k, soff, 0));
    w[k] = v.x; w[k + 1] = v.y;
  } else if constexpr (N % 4 == 1) {
    w[k] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4u * k, soff, 0);
  }
}

// Shift N words right by sh bits (0..31) as one little-endian bit string, so
// that the window's first code starts at bit 0.
template <int N>
__device__ __forceinline__ void align_words(uint32_t* w, uint32_t sh) {
#pragma unroll
  for (int k = 0; k + 1 < N; ++k) w[k] = __builtin_amdgcn_alignbit(w[k + 1], w[k], sh);
  w[N - 1] = __builtin_amdgcn_alignbit(0u, w[N - 1], sh);
}

// Chunk at byte `off` (chunk_byte) of the buffer.
template <int B>
__device__ __forceinline__ void load_chunk(Chunk<B>& c, rsrc_t r, uint32_t off) {
  if constexpr (B == 8) {
    u32x4 v = buf_load_b128(r, off);  // 16-byte aligned
    c.w[0] = v.x; c.w[1] = v.y; c.w[2] = v.z; c.w[3] = v.w;
  } else if constexpr (B == 12) {
    u32x2 a = buf_load_b64(r, off);   // 24 bytes on an 8-byte boundary
    u32x2 b = buf_load_b64(r, off + 8);
    u32x2 d = buf_load_b64(r, off + 16);
    c.w[0] = a.x; c.w[1] = a.y; c.w[2] = b.x; c.w[3] = b.y; c.w[4] = d.x; c.w[5] = d.y;
  } else {
    load_words<Chunk<B>::kWords>(c.w, r, off);
  }
}

// Chunk q of a row whose words start at p (any width; shifted into place).
template <int B>
__device__ __forceinline__ void load_chunk(Chunk<B>& c, const uint32_t* row, uint32_t q) {
  const uint32_t* p = row + chunk_byte<B>(q) / 4;
  if constexpr (B == 8) {
    u32x4 v = *reinterpret_cast<const u32x4*>(p);  // 16-byte aligned
    c.w[0] = v.x; c.w[1] = v.y; c.w[2] = v.z; c.w[3] = v.w;
  } else if constexpr (B == 12) {
    // 24 bytes on an 8-byte boundary
    u32x2 a = *reinterpret_cast<const u32x2*>(p);
    u32x2 b = *reinterpret_cast<const u32x2*>(p + 2);
    u32x2 d = *reinterpret_cast<const u32x2*>(p + 4);
    c.w[0] = a.x; c.w[1] = a.y; c.w[2] = b.x; c.w[3] = b.y; c.w[4] = d.x; c.w[5] = d.y;
  } else {
#pragma unroll
    for (int k = 0; k < Chunk<B>::kWords; ++k) c.w[k] = p[k];
    if constexpr (B & 1) align_words<Chunk<B>::kWords>(c.w, chunk_shift<B>(q));
  }
}

// Bring a chunk loaded at chunk_byte(q) into place (odd widths, odd q).
template <int B>
__device__ __forceinline__ void align_chunk(Chunk<B>& c, uint32_t sh) {
  if constexpr ((B & 1) && !kAlignedChunks<B>) align_words<Chunk<B>::kWords>(c.w, sh);
}

// Code i (0..15, compile-time after unrolling) of a chunk.
template <int B>
__device__ __forceinline__ uint32_t chunk_code(const Chunk<B>& c, int i) {
  constexpr uint32_t mask = (1u << B) - 1u;
  const int bit = i * B;
  const int wi = bit >> 5;
  const int sh = bit & 31;
  if (sh + B <= 32) return (c.w[wi] >> sh) & mask;
  return __builtin_amdgcn_alignbit(c.w[wi + 1], c.w[wi], sh) & mask;  // straddles two words
}

// ---------------------------------------------------------------------------
// codebook in LDS
// ---------------------------------------------------------------------------
//
// Two layouts.
//
// Replicated (K = 256 only): each 256-byte LDS row holds 128/D copies of one
// entry side by side, so the byte offset of copy c of entry e is
//   e * 256 + c * (2*D).
// A lane always reads copy (lane % copies): the LDS bank it touches depends
// only on its lane id, never on the code, so a wave's random gather is free of
// bank conflicts (64 lanes x 4 B, 32 lanes x 8 B or 16 lanes x 16 B hit
// pairwise different banks within each LDS cycle).  The offset is one
// v_perm_b32: byte 1 = the 8-bit code, byte 0 = the lane's copy offset.
// 64 KiB for every D.
//
// Plain (any K): entry e at e * (2*D) bytes; random gathers may conflict.
// Used for every other K whose codebook takes at most 64 KiB (K = 4096: 16,
// 32 and 64 KiB for d = 2, 4, 8; K = 16384 at d = 2: 64 KiB).
//
// Device memory (codebooks above 64 KiB: d = 4 with K = 16384, d = 8 with K =
// 8192 or 16384): not staged; each gather reads the entry from the codebook
// in device memory, where it stays resident in the L2 caches.  The slower
// path, as the paper's device-memory codebook variant (§3.4), for the
// codebooks that do not fit next to the kernels' other LDS buffers.

template <int D, int B>
struct CodebookLayout {
  static constexpr int kEntryBytes = 2 * D;
  static constexpr bool kReplicated = (B == 8);
  static constexpr bool kGlobal = !kReplicated && (1 << B) * kEntryBytes > 64 * 1024;
  static constexpr int kCopies = kReplicated ? 256 / kEntryBytes : 1;
  static constexpr int kBytes = kReplicated ? 256 * 256 : (kGlobal ? 16 : (1 << B) * kEntryBytes);
};

// Stage `cb` (global, [K][D] fp16, 16-byte aligned) into `lds`.
// All threads of the block take part; the caller synchronises afterwards.
// Every thread issues all of its global loads before its first LDS write, so
// the staging costs one round trip to L2 rather than one per slot.
template <int D, int B>
__device__ __forceinline__ void stage_codebook(uint8_t* lds, const uint16_t* cb, int tid,
                                               int nthreads) {
  using L = CodebookLayout<D, B>;
  if constexpr (L::kGlobal) {
    return;  // gathered from device memory
  } else if constexpr (L::kReplicated) {
    // 4096 slots of 16 bytes; slot q holds copies of entry q / 16.  Lanes
    // write consecutive slots (conflict-free); the 16 lanes sharing an entry
    // read the same global address (one L1 line).
    constexpr int V = 8;
    for (int base = tid; base < 4096; base += V * nthreads) {
      u32x4 v[V];
#pragma unroll
      for (int u = 0; u < V; ++u) {
        const int q = base + u * nthreads;
        const int e = (q < 4096 ? q : 0) >> 4;
        if constexpr (D == 2) {
          const uint32_t a = reinterpret_cast<const uint32_t*>(cb)[e];
          v[u] = u32x4{a, a, a, a};
        } else if constexpr (D == 4) {
          const u32x2 a = reinterpret_cast<const u32x2*>(cb)[e];
          v[u] = u32x4{a.x, a.y, a.x, a.y};
        } else {
          v[u] = reinterpret_cast<const u32x4*>(cb)[e];
        }
      }
#pragma unroll
      for (int u = 0; u < V; ++u) {
        const int q = base + u * nthreads;
        if (q < 4096) reinterpret_cast<u32x4*>(lds)[q] = v[u];
      }
    }
  } else {
    constexpr int n16 = L::kBytes / 16;
    constexpr int V = 8;
    for (int base = tid; base < n16; base += V * nthreads) {
      u32x4 v[V];
#pragma unroll
      for (int u = 0; u < V; ++u) {
        const int q = base + u * nthreads;
        v[u] = reinterpret_cast<const u32x4*>(cb)[q < n16 ? q : 0];
      }
#pragma unroll
      for (int u = 0; u < V; ++u) {
        const int q = base + u * nthreads;
        if (q < n16) reinterpret_cast<u32x4*>(lds)[q] = v[u];
      }
    }
  }
}

// Per-lane constant part of the gather offset (replicated layout).
template <int D, int B>
__device__ __forceinline__ uint32_t lane_copy_offset(int lane) {
  using L = CodebookLayout<D, B>;
  if constexpr (L::kReplicated) return (uint32_t)((lane % L::kCopies) * L::kEntryBytes);
  return 0u;
}

// Byte offset in LDS of entry `code` for this lane.  For the replicated
// layout `word` is the packed word holding the 8-bit code as byte `byte`.
template <int D, int B>
__device__ __forceinline__ uint32_t entry_offset_byte(uint32_t word, int byte, uint32_t lane_off) {
  // v_perm_b32: result byte0 = lane_off byte0, byte1 = word byte `byte`, bytes 2-3 = 0
  const uint32_t sel = 0x0C0C0000u | ((uint32_t)(4 + byte) << 8);
  return __builtin_amdgcn_perm(word, lane_off, sel);
}

template <int D>
struct Entry;
template <> struct Entry<2> { half2_t v[1]; };
template <> struct Entry<4> { half2_t v[2]; };
template <> struct Entry<8> { half2_t v[4]; };

// The d fp16 values of the entry at byte `off` of the codebook at `lds` (LDS,
// or device memory for the large codebooks).
template <int D>
__device__ __forceinline__ Entry<D> lds_entry(const uint8_t* lds, uint32_t off) {
  Entry<D> e;
  if constexpr (D == 2) {
    e.v[0] = *reinterpret_cast<const half2_t*>(lds + off);
  } else if constexpr (D == 4) {
    half4_t h = *reinterpret_cast<const half4_t*>(lds + off);
    e.v[0] = half2_t{h.x, h.y};
    e.v[1] = half2_t{h.z, h.w};
  } else {
    half8_t h = *reinterpret_cast<const half8_t*>(lds + off);
    e.v[0] = half2_t{h[0], h[1]};
    e.v[1] = half2_t{h[2], h[3]};
    e.v[2] = half2_t{h[4], h[5]};
    e.v[3] = half2_t{h[6], h[7]};
  }
  return e;
}

// Entry of code i of a chunk for this lane.
template <int D, int B>
__device__ __forceinline__ Entry<D> gather(const uint8_t* lds, const Chunk<B>& c, int i,
                                           uint32_t lane_off) {
  using L = CodebookLayout<D, B>;
  uint32_t off;
  if constexpr (L::kReplicated) {
    off = entry_offset_byte<D, B>(c.w[i >> 2], i & 3, lane_off);
  } else {
    off = chunk_code<B>(c, i) * (uint32_t)L::kEntryBytes;
  }
  return lds_entry<D>(lds, off);
}

__device__ __forceinline__ half2_t as_half2(uint32_t u) {
  return __builtin_bit_cast(half2_t, u);
}
__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ float dot2(half2_t a, half2_t b, float c) {
  return __builtin_amdgcn_fdot2(a, b, c, false);  // v_dot2_f32_f16
}

// Sum over each 16-lane DPP row; every lane of the row gets the total.
// quad_perm [1,0,3,2] and [2,3,0,1] sum each quad, row_half_mirror pairs the
// two quads of each half-row, row_mirror pairs the two half-rows.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);  // row_half_mirror
  v += dpp_mov<0x140>(v);  // row_mirror
  return v;
}

// Block barrier that orders LDS only: waits for this wave's LDS operations,
// not for its global loads in flight, so a prefetch issued before the
// barrier stays in flight across it.  (hipcc's __syncthreads compiles to the
// same two instructions for gfx950; spelling them out keeps that property
// from depending on how the compiler lowers the fence.)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// ---------------------------------------------------------------------------
// input / output conversions and the fused output step
// ---------------------------------------------------------------------------

// Two bf16 values (low half first) to two fp16 values, round to nearest even:
// a bf16 value widens to fp32 exactly, and fp32 -> fp16 rounds once.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  const float lo = __builtin_bit_cast(float, w << 16);
  const float hi = __builtin_bit_cast(float, w & 0xffff0000u);
  return as_u32(half2_t{(_Float16)lo, (_Float16)hi});
}
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
  return u32x4{bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z), bf16x2_to_f16x2(v.w)};
}

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// y[i] = v in the output type (0 fp32, 1 fp16, 2 bf16; round to nearest even).
__device__ __forceinline__ void store_out(void* out, int64_t i, float v, int kind) {
  if (kind == 0) reinterpret_cast<float*>(out)[i] = v;
  else if (kind == 1) reinterpret_cast<_Float16*>(out)[i] = (_Float16)v;
  else reinterpret_cast<uint16_t*>(out)[i] = f32_to_bf16_bits(v);
}

// SwiGLU gate: silu(g) * u with silu(g) = g / (1 + exp(-g)).
__device__ __forceinline__ float swiglu(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

}  // namespace vqmi
