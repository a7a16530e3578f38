// kp_read_rows: a read-only row gather, the bandwidth reference for the attention's own access pattern.
//
// The attention stage gathers whole 1 KiB value rows of the selected tokens from the paged latent cache.  This
// kernel reads a given list of rows the same way -- one wave-wide 16-byte direct load per 1 KiB of row, straight
// into LDS, rows taken in list order in contiguous runs per wave -- and discards them: no compute, no barrier, no
// output.  Timed over the attention's own row list it measures what HBM delivers for that pattern on this machine,
// the practical ceiling the attention kernel is compared with.
//
// Grid: 256 threads (4 waves) per block, two blocks per compute unit (scaled by the caller's block count); each wave
// takes a contiguous run of the list and keeps two groups of 4 rows in flight (double-buffered in its own LDS area).
#include "kp_device.hpp"
#include "kp_internal.hpp"

namespace kp {

constexpr int RR_THREADS = 256;
constexpr int RR_GROUP = 4;  // rows per group; two groups in flight per wave

template <int CH>  // 1 KiB units per row
__global__ __launch_bounds__(RR_THREADS) void read_rows_kernel(const char* __restrict__ base, int64_t row_stride,
                                                               const int32_t* __restrict__ rows, int64_t n_rows) {
  __shared__ __align__(1024) char lds[RR_THREADS / 64][2][RR_GROUP][1024];  // a row's units share its slot
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int64_t wave = int64_t(blockIdx.x) * (RR_THREADS / 64) + wv;
  const int64_t n_waves = int64_t(gridDim.x) * (RR_THREADS / 64);
  const int64_t per = (n_rows + n_waves - 1) / n_waves;
  const int64_t r_begin = wave * per;
  const int64_t r_end = r_begin + per < n_rows ? r_begin + per : n_rows;
  if (r_begin >= r_end) return;
  const uint32_t my = lds_off(&lds[wv][0][0][0]);
  int g = 0;
  for (int64_t r0 = r_begin; r0 < r_end; r0 += RR_GROUP, ++g) {
    int idx[RR_GROUP];
#pragma unroll
    for (int u = 0; u < RR_GROUP; ++u) idx[u] = rows[r0 + u < r_end ? r0 + u : r_begin];  // uniform: scalar loads
#pragma unroll
    for (int u = 0; u < RR_GROUP; ++u) {
      const char* row = base + int64_t(__builtin_amdgcn_readfirstlane(idx[u])) * row_stride;
#pragma unroll
      for (int c = 0; c < CH; ++c)  // 1 KiB per wave load
        lds_dma16(row + c * 1024 + lane * 16, my + uint32_t(((g & 1) * RR_GROUP + u) * 1024));
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(RR_GROUP * CH));  // the older group has landed
  }
  __builtin_amdgcn_s_waitcnt(0);  // nothing may land in LDS after the block ends
}

kp_status launch_read_rows(const void* base, int64_t row_stride, int32_t row_bytes, const int32_t* rows,
                           int64_t n_rows, int blocks, hipStream_t s) {
  if (n_rows == 0) return KP_OK;
  const char* b = static_cast<const char*>(base);
  if (row_bytes == 4096)
    read_rows_kernel<4><<<dim3(unsigned(blocks)), dim3(RR_THREADS), 0, s>>>(b, row_stride, rows, n_rows);
  else
    read_rows_kernel<1><<<dim3(unsigned(blocks)), dim3(RR_THREADS), 0, s>>>(b, row_stride, rows, n_rows);
  return check_launch("kp_read_rows");
}

}  // namespace kp
