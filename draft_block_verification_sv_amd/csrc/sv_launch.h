// Kernel argument blocks and the internal (C++) launch functions the C ABI calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_layout.h"

namespace sv {

struct PlanArgs {
  int64_t B;
  int32_t k_max;
  int64_t V;
  int64_t n_d;
  const int32_t* k;
  const int32_t* tokens;
  const float* uniforms;
  const float* temperature;  // nullable
  Workspace ws;
  int32_t* device_status;
};

struct RowsArgs {
  const void* target;
  const void* draft;
  int64_t ld_t, ld_d;
  int32_t V;
  int64_t n_slices;
  int64_t n_waves;            // n_units * n_slices (< 2^31)
  const RowDesc* desc;        // verification: per target row; nullptr for rKL only
  const int32_t* glob;        // verification: void flag
  const int32_t* p_row_index; // rKL only (nullable = identity)
  int64_t n_target_rows;      // rKL only: bound for p_row_index
  int32_t* device_status;     // rKL only: reset by the first wave
  Partials part;
};

struct FinArgs {
  const void* target;
  const void* draft;
  int64_t ld_t, ld_d;
  int32_t V;
  int64_t n_slices;
  int64_t n_units;
  int64_t n_d;
  const RowDesc* desc;  // nullptr for rKL only
  const int32_t* glob;
  const int32_t* req_flags;
  const int32_t* tokens;
  const float* uniforms;
  const int32_t* p_row_index;
  int64_t n_target_rows;
  int32_t* device_status;
  Partials part;
  float delta;
  float* rkl_out;  // nullable in verification
  float* p_at;     // nullable
  float* q_at;     // nullable
  float* t_off;
  float* t_lz;
  int32_t* t_arg;
  float* d_off;
  float* d_lz;
  int32_t* acc;
};

struct SampleArgs {
  const void* target;
  const void* draft;
  int64_t ld_t, ld_d;
  int32_t V;
  int64_t n_chunks;
  int64_t B;
  int64_t n_t;
  const int32_t* glob;
  const int32_t* off_t;
  const int32_t* k;
  const int32_t* req_flags;
  const RowDesc* desc;
  const int32_t* tokens;
  const float* uniforms;
  const float* t_off;
  const float* t_lz;
  const int32_t* t_arg;
  const float* d_off;
  const float* d_lz;
  const int32_t* acc;
  double* chunk_r;
  double* chunk_p;
  int32_t* accept_len;
  int32_t* out_tokens;
};

hipError_t launch_plan(const PlanArgs& a, hipStream_t st);
hipError_t launch_rows(int dtype, bool vec, const RowsArgs& a, hipStream_t st);
hipError_t launch_finalize(int dtype, const FinArgs& a, hipStream_t st);
hipError_t launch_sample_chunks(int dtype, bool vec, const SampleArgs& a, hipStream_t st);
hipError_t launch_sample_finish(int dtype, bool vec, const SampleArgs& a, hipStream_t st);

}  // namespace sv
