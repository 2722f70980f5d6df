// Inverted lists of a soft assignment from the selections of every row at
// once (gfx950): a stable radix sort of (list, row) pairs.
//
// Method: "Flash-GMM: A Memory-Efficient Kernel for Scalable Soft Clustering",
// Section 4.2 / 4.3 (each vector is appended to the inverted list of each
// component it is assigned to; the lists then serve an IVF index).
//
// The selections sel[row * stride + j] (component id, -1 = none) are laid out
// in row order, so sorting the entries by component with a stable sort leaves
// the rows of each list in ascending order: the same lists as the chunked
// count / scan / scatter path, built in a few device-wide passes instead of
// one thread per row block.  Entries with no component get the key K and sort
// to the end; the first nnz sorted rows are the list ids.
#include <hipcub/hipcub.hpp>

#include "gmm_internal.h"

namespace gmm {

// keys[i] = the component of entry i (K for none), rows[i] = its row.
__global__ void k_list_pairs(const int32_t* __restrict__ sel, int64_t n, int stride, unsigned none,
                             unsigned* __restrict__ keys, int32_t* __restrict__ rows) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int k = sel[i];
    keys[i] = (k < 0) ? none : (unsigned)k;
    rows[i] = (int32_t)(i / stride);
  }
}

static int key_bits(int K) {
  int b = 1;
  while ((1u << b) <= (unsigned)K) ++b;  // keys 0..K
  return b;
}

static size_t up256(size_t b) { return (b + 255) / 256 * 256; }

size_t sort_lists_bytes(int64_t n, int K) {
  size_t temp = 0;
  const int bits = key_bits(K);
  if (hipcub::DeviceRadixSort::SortPairs(nullptr, temp, (const unsigned*)nullptr, (unsigned*)nullptr,
                                         (const int32_t*)nullptr, (int32_t*)nullptr, (int)n, 0, bits) !=
      hipSuccess)
    return 0;
  return 4 * up256((size_t)n * 4) + up256(temp);
}

hipError_t sort_lists(const int32_t* sel, int64_t rows, int stride, int K, int32_t* ids, int64_t nnz, void* buf,
                      size_t bytes, hipStream_t s) {
  const int64_t n = rows * stride;
  if (n <= 0) return hipSuccess;
  if (n > INT32_MAX) return hipErrorInvalidValue;
  const int bits = key_bits(K);
  char* q = static_cast<char*>(buf);
  unsigned* kin = reinterpret_cast<unsigned*>(q);
  q += up256((size_t)n * 4);
  unsigned* kout = reinterpret_cast<unsigned*>(q);
  q += up256((size_t)n * 4);
  int32_t* vin = reinterpret_cast<int32_t*>(q);
  q += up256((size_t)n * 4);
  int32_t* vout = reinterpret_cast<int32_t*>(q);
  q += up256((size_t)n * 4);
  size_t temp = bytes - (size_t)(q - static_cast<char*>(buf));
  size_t need = 0;
  hipError_t e = hipcub::DeviceRadixSort::SortPairs(nullptr, need, (const unsigned*)kin, kout, (const int32_t*)vin,
                                                    vout, (int)n, 0, bits, s);
  if (e != hipSuccess) return e;
  if (need > temp) return hipErrorInvalidValue;
  size_t g = (size_t)((n + 255) / 256);
  if (g > 65535 * 4) g = 65535 * 4;
  hipLaunchKernelGGL(k_list_pairs, dim3((unsigned)g), dim3(256), 0, s, sel, n, stride, (unsigned)K, kin, vin);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipcub::DeviceRadixSort::SortPairs((void*)q, temp, (const unsigned*)kin, kout, (const int32_t*)vin, vout,
                                         (int)n, 0, bits, s);
  if (e != hipSuccess) return e;
  if (nnz > 0) e = hipMemcpyAsync(ids, vout, (size_t)nnz * 4, hipMemcpyDeviceToDevice, s);
  return e;
}

}  // namespace gmm
