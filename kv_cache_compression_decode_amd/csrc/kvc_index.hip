// Bitstream index: every (chunk, layer, K/V, channel) stream's block offset,
// the exclusive prefix sum of the stream lengths rounded up to whole 8-byte
// blocks in (layer, K/V, channel) order (a unit's payload starts at its
// first stream's offset), plus container header validation.
//
// Two launches over a (row = layer*2 + kv, chunk) grid:
//   k_index_rows : per row, the sum of padded lengths (u64); the row-0 block
//                  validates the chunk's header against the descriptor and
//                  the tables' profile id;
//   k_index_scan : per row, the base offset (sum of earlier rows) and a block
//                  scan of the row's C lengths; the last row checks that the
//                  total equals the header's payload size and that the
//                  container size adds up, and marks the chunk decodable.
// The decoder only touches chunks marked valid, so a corrupt container can
// never send it outside the container.
#include "kvc_internal.h"

namespace kvc {

__device__ inline uint32_t ld_u32(const uint8_t *p) {
  // 4-byte aligned by construction (containers start 4-aligned, records are 16 B)
  return *reinterpret_cast<const uint32_t *>(p);
}
__device__ inline uint64_t ld_u64(const uint8_t *p) {
  return (uint64_t)ld_u32(p) | ((uint64_t)ld_u32(p + 4) << 32);
}

__global__ void k_load_chunks(ChunkBatch batch, ChunkInfo *dst, uint32_t *flags, uint32_t first,
                              uint32_t count) {
  const uint32_t i = threadIdx.x;
  if (i < count) {
    dst[first + i] = batch.c[i];
    flags[first + i] = 0;
  }
}

// Per-chunk problem flags, OR-ed by the row blocks.
constexpr uint32_t kFlagHeader = 1u;  // header does not match descriptor / tables
constexpr uint32_t kFlagShort = 2u;   // a stream shorter than its 4 flush bytes

__global__ void k_reset_status(int32_t *status) {
  if (threadIdx.x == 0) *status = 0;
}

__device__ int32_t check_header(const Desc &d, const ChunkInfo &ci, const uint8_t *tables) {
  const uint8_t *h = ci.cont;
  if (ld_u32(h) != kContainerMagic) return KVC_ERR_CORRUPT_STREAM;
  const uint32_t w1 = ld_u32(h + 4);  // version u16, level u8, anchor_bits u8
  if ((w1 & 0xFFFFu) != kFormatVersion) return KVC_ERR_CORRUPT_STREAM;
  const uint32_t level = (w1 >> 16) & 0xFFu;
  if (level != ci.level || ((w1 >> 24) & 0xFFu) != 8u) return KVC_ERR_CORRUPT_STREAM;
  const uint32_t w2 = ld_u32(h + 8);  // group u16, prec u8, bits[0] u8
  const uint32_t w3 = ld_u32(h + 12); // bits[1] u8, bits[2] u8, reserved u16
  if ((w2 & 0xFFFFu) != d.G || ((w2 >> 16) & 0xFFu) != kPrec) return KVC_ERR_CORRUPT_STREAM;
  if (level >= d.nlev) return KVC_ERR_CORRUPT_STREAM;
  if (((w2 >> 24) & 0xFFu) != d.bits[level][0] || (w3 & 0xFFu) != d.bits[level][1] ||
      ((w3 >> 8) & 0xFFu) != d.bits[level][2])
    return KVC_ERR_CORRUPT_STREAM;
  if (ld_u32(h + 16) != d.L || ld_u32(h + 20) != d.C) return KVC_ERR_CORRUPT_STREAM;
  if (ld_u32(h + 24) != ci.n_tokens) return KVC_ERR_CORRUPT_STREAM;
  if (ld_u32(h + 48) != d.chunk || ld_u32(h + 52) != n_streams(d)) return KVC_ERR_CORRUPT_STREAM;
  const uint64_t pid = ld_u64(h + 32);
  const uint64_t tpid = *reinterpret_cast<const uint64_t *>(tables + 48);
  if (pid != tpid) return KVC_ERR_PROFILE_MISMATCH;
  return KVC_OK;
}

// A refinement container ("KVCR") against the descriptor and the refinement
// tables (its E, its id and the base profile id they were made for).
__device__ int32_t check_refine_header(const Desc &d, const ChunkInfo &ci, const uint8_t *rtables) {
  const uint8_t *h = ci.cont;
  if (ld_u32(h) != kRefineContainerMagic) return KVC_ERR_CORRUPT_STREAM;
  const uint32_t w1 = ld_u32(h + 4);  // version u16, level u8, E u8
  if ((w1 & 0xFFFFu) != kRefineVersion) return KVC_ERR_CORRUPT_STREAM;
  const uint32_t level = (w1 >> 16) & 0xFFu;
  if (level != ci.level || level >= d.nlev) return KVC_ERR_CORRUPT_STREAM;
  if (((w1 >> 24) & 0xFFu) != ld_u32(rtables + 24)) return KVC_ERR_CORRUPT_STREAM;
  const uint32_t w2 = ld_u32(h + 8);
  const uint32_t w3 = ld_u32(h + 12);
  if ((w2 & 0xFFFFu) != d.G || ((w2 >> 16) & 0xFFu) != kPrec) return KVC_ERR_CORRUPT_STREAM;
  if (((w2 >> 24) & 0xFFu) != d.bits[level][0] || (w3 & 0xFFu) != d.bits[level][1] ||
      ((w3 >> 8) & 0xFFu) != d.bits[level][2])
    return KVC_ERR_CORRUPT_STREAM;
  if (ld_u32(h + 16) != d.L || ld_u32(h + 20) != d.C) return KVC_ERR_CORRUPT_STREAM;
  if (ld_u32(h + 24) != ci.n_tokens) return KVC_ERR_CORRUPT_STREAM;
  if (ld_u32(h + 48) != d.chunk || ld_u32(h + 52) != n_streams(d)) return KVC_ERR_CORRUPT_STREAM;
  if (ld_u64(h + 32) != ld_u64(rtables + 48) || ld_u64(h + 56) != ld_u64(rtables + 56))
    return KVC_ERR_PROFILE_MISMATCH;
  return KVC_OK;
}

__global__ __launch_bounds__(256) void k_index_rows(Desc d, const ChunkInfo *__restrict__ ci,
                                                    uint64_t *__restrict__ row_sums,
                                                    uint32_t *__restrict__ flags,
                                                    const uint8_t *__restrict__ tables,
                                                    int check_header_flag, int32_t *status) {
  const uint32_t row = blockIdx.x, k = blockIdx.y;
  const uint32_t nrows = 2u * d.L;
  const ChunkInfo c = ci[k];
  const uint8_t *rec = c.records + (uint64_t)row * d.C * kRecBytes;
  uint64_t acc = 0;
  bool short_stream = false;
  for (uint32_t ch = threadIdx.x; ch < d.C; ch += blockDim.x) {
    const uint32_t nb = ld_u32(rec + (uint64_t)ch * kRecBytes + 12);
    short_stream = short_stream || nb < 4u;
    acc += pad8(nb);
  }
  // block reduction
  __shared__ uint64_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (uint32_t s = blockDim.x / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (check_header_flag && __syncthreads_or(short_stream) && threadIdx.x == 0) {
    atomicOr(&flags[k], kFlagShort);
    set_status(status, KVC_ERR_CORRUPT_STREAM);
  }
  if (threadIdx.x == 0) {
    row_sums[(uint64_t)k * nrows + row] = red[0];
    if (row == 0 && check_header_flag) {
      // 1: a base container against the tables; 2: a refinement container
      // against the refinement tables
      const int32_t st =
          check_header_flag == 2 ? check_refine_header(d, c, tables) : check_header(d, c, tables);
      if (st != KVC_OK) {
        atomicOr(&flags[k], kFlagHeader);
        set_status(status, st);
      }
    }
  }
}

// Inclusive scan of one value per thread over a 256-thread block.
__device__ inline uint64_t block_scan_incl(uint64_t v, uint64_t *tmp) {
  const uint32_t t = threadIdx.x;
  tmp[t] = v;
  __syncthreads();
  for (uint32_t off = 1; off < blockDim.x; off <<= 1) {
    const uint64_t add = t >= off ? tmp[t - off] : 0;
    __syncthreads();
    tmp[t] += add;
    __syncthreads();
  }
  const uint64_t r = tmp[t];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(256) void k_index_scan(Desc d, const ChunkInfo *__restrict__ ci,
                                                    const uint64_t *__restrict__ row_sums,
                                                    const uint32_t *__restrict__ flags,
                                                    uint32_t *__restrict__ offsets,
                                                    uint8_t *__restrict__ valid,
                                                    uint64_t *__restrict__ payload,
                                                    int check_header_flag, int32_t *status) {
  const uint32_t row = blockIdx.x, k = blockIdx.y;
  const uint32_t nrows = 2u * d.L;
  const uint32_t S = n_streams(d);
  const ChunkInfo c = ci[k];
  __shared__ uint64_t tmp[256];
  __shared__ uint64_t base_sh;
  if (threadIdx.x == 0) {
    uint64_t b = 0;
    for (uint32_t r = 0; r < row; ++r) b += row_sums[(uint64_t)k * nrows + r];
    base_sh = b;
  }
  __syncthreads();
  uint64_t running = base_sh;
  const uint8_t *rec = c.records + (uint64_t)row * d.C * kRecBytes;
  uint32_t *out = offsets + (uint64_t)k * S + (uint64_t)row * d.C;
  for (uint32_t t0 = 0; t0 < d.C; t0 += blockDim.x) {
    const uint32_t ch = t0 + threadIdx.x;
    const uint64_t v = ch < d.C ? pad8(ld_u32(rec + (uint64_t)ch * kRecBytes + 12)) : 0;
    const uint64_t incl = block_scan_incl(v, tmp);
    if (ch < d.C) out[ch] = (uint32_t)(running + incl - v);
    // the tile's total is the last thread's inclusive value
    const uint64_t tile_total = tmp[blockDim.x - 1];
    __syncthreads();
    running += tile_total;
  }
  if (row == nrows - 1 && threadIdx.x == 0) {
    const uint64_t total = running;
    payload[k] = total;
    uint8_t ok = 1;
    if (check_header_flag) {
      ok = flags[k] == 0;
      if (ok) {
        const uint64_t hp = ld_u64(c.cont + 40);
        const uint64_t want = (uint64_t)kHdrBytes + (uint64_t)kRecBytes * S + total;
        // every stream offset must fit in 32 bits
        if (hp != total || c.cont_bytes != want || total > 0xFFFFFFFFull) {
          ok = 0;
          set_status(status, KVC_ERR_CORRUPT_STREAM);
        }
      }
    }
    valid[k] = ok;
  }
}

// Host launchers shared by decode and encode.  The chunk table travels as
// kernel arguments, so the caller's host array may be released at once.
hipError_t launch_load_chunks(const ChunkInfo *host_chunks, uint32_t n_chunks,
                              ChunkInfo *dev_chunks, uint32_t *flags, hipStream_t stream) {
  for (uint32_t first = 0; first < n_chunks; first += kMaxChunksPerBatch) {
    const uint32_t count =
        n_chunks - first < kMaxChunksPerBatch ? n_chunks - first : kMaxChunksPerBatch;
    ChunkBatch b;
    for (uint32_t i = 0; i < count; ++i) b.c[i] = host_chunks[first + i];
    hipLaunchKernelGGL(k_load_chunks, dim3(1), dim3(kMaxChunksPerBatch), 0, stream, b,
                       dev_chunks, flags, first, count);
  }
  return hipGetLastError();
}

__global__ void k_load_groups(GroupBatch batch, DecodeGroup *dst, uint32_t first, uint32_t count) {
  const uint32_t i = threadIdx.x;
  if (i < count) dst[first + i] = batch.g[i];
}

hipError_t launch_load_groups(const DecodeGroup *host_groups, uint32_t n_groups,
                              DecodeGroup *dev_groups, hipStream_t stream) {
  for (uint32_t first = 0; first < n_groups; first += kMaxChunksPerBatch) {
    const uint32_t count =
        n_groups - first < kMaxChunksPerBatch ? n_groups - first : kMaxChunksPerBatch;
    GroupBatch b;
    for (uint32_t i = 0; i < count; ++i) b.g[i] = host_groups[first + i];
    hipLaunchKernelGGL(k_load_groups, dim3(1), dim3(kMaxChunksPerBatch), 0, stream, b,
                       dev_groups, first, count);
  }
  return hipGetLastError();
}

hipError_t launch_index(const Desc &d, const ChunkInfo *dev_chunks, uint32_t n_chunks,
                        uint64_t *row_sums, uint32_t *flags, uint32_t *offsets, uint8_t *valid,
                        uint64_t *payload, const uint8_t *tables, int check_header_flag,
                        int32_t *status, hipStream_t stream) {
  const dim3 grid(2u * d.L, n_chunks);
  hipLaunchKernelGGL(k_index_rows, grid, dim3(256), 0, stream, d, dev_chunks, row_sums, flags,
                     tables, check_header_flag, status);
  hipLaunchKernelGGL(k_index_scan, grid, dim3(256), 0, stream, d, dev_chunks, row_sums, flags,
                     offsets, valid, payload, check_header_flag, status);
  return hipGetLastError();
}

hipError_t launch_reset_status(int32_t *status, hipStream_t stream) {
  hipLaunchKernelGGL(k_reset_status, dim3(1), dim3(64), 0, stream, status);
  return hipGetLastError();
}

}  // namespace kvc
