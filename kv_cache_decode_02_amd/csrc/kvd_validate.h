// Host-side precondition checks of the C ABI (validate.cpp), used by the
// entry points when KVD_VALIDATE=1.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace kvd {

// Host-side precondition checks (validate.cpp).  DeviceChecks names device
// arrays; validate_device copies them to the host on `stream`, synchronises
// and checks: 1 <= seq_lens[b] <= min(max_seq_len, MB * 16) (max_seq_len 0:
// MB * 16), every table entry of a visible block inside [0, num_blocks), the
// blocks that receive new rows (the last position when writes_last, the
// rows of cu_rows when given) owned by that sequence alone, and finite values
// in the listed small arrays.
struct FiniteCheck {
  const void* ptr;
  size_t bytes;
  int dtype;
};
struct DeviceChecks {
  const int32_t* seq_lens;
  const int32_t* block_table;
  const int32_t* cu_rows;  // [B + 1] row offsets of a multi-row append, or NULL
  int batch, max_blocks_per_seq, num_blocks, max_seq_len;
  bool writes_last;
  FiniteCheck finite[3];
  int num_finite;
};
int validate_tables(const int32_t* seq_lens, const int32_t* block_table, int batch,
                    int max_blocks_per_seq, int num_blocks, int max_seq_len,
                    const int32_t* new_rows, int* first_bad);
int validate_finite(const void* data, size_t count, int dtype);
bool validation_enabled();  // KVD_VALIDATE=1 in the environment
int validate_device(const DeviceChecks& c, hipStream_t stream);

}  // namespace kvd
