// Plan-time sort for the transposed plan: a stable device radix sort
// (rocPRIM's) of the column indices carrying each entry's position. It runs
// once per plan, never in spmv_exec.
#include <cstring>

#include <rocprim/device/device_radix_sort.hpp>
#include <rocprim/iterator/counting_iterator.hpp>

#include "internal.hpp"

namespace spmv {

hipError_t sort_columns(void* temp, size_t* temp_bytes, const int32_t* keys, int32_t* keys_out,
                        int32_t* perm_out, int64_t nnz, int bits, hipStream_t s) {
  rocprim::counting_iterator<int32_t> position(0);
  return rocprim::radix_sort_pairs(temp, *temp_bytes, keys, keys_out, position, perm_out,
                                   (size_t)nnz, 0u, (unsigned)bits, s);
}

}  // namespace spmv
