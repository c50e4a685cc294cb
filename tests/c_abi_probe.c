/* A plain C99 consumer of include/pkv.h and the shared library, built with
 * gcc by tests/test_c_abi.py.  It prints, one "key value..." per line, the
 * layout of the public structures, the constants, the host-only entry points'
 * results for a few problems and their argument checks; the test compares
 * them with the Python binding's ctypes view.  No GPU call is made: every
 * plan is asked for an explicit compute-unit count. */
#include <stddef.h>
#include <stdio.h>
#include <string.h>

#include "pkv.h"

static pkv_problem decode_problem(void) {
  pkv_problem p;
  memset(&p, 0, sizeof p);
  p.batch = 8;
  p.q_len = 1;
  p.num_q_heads = 24;
  p.num_kv_heads = 4;
  p.head_dim = 64;
  p.page_size = 32;
  p.num_pages = 512;
  p.max_pages_per_seq = 64;
  p.max_kv_len = 2048;
  p.scale = 0.125f;
  p.causal_offset = -1;
  return p;
}

static void print_plan(const char *tag, int rc, const pkv_plan_info *i) {
  printf("%s %d %d %d %d %d %lld %lld %d %d %d %d\n", tag, rc, i->splits, i->heads_per_block, i->rows_per_block,
         i->matrix_core, (long long)i->units, (long long)i->workgroups, i->merge_in_kernel, i->kernels, i->kernel,
         i->paired_heads);
}

#define FIELD(T, f) printf("offset " #T " " #f " %zu %zu\n", offsetof(T, f), sizeof(((T *)0)->f))

int main(void) {
  printf("sizeof pkv_problem %zu\n", sizeof(pkv_problem));
  printf("sizeof pkv_plan_info %zu\n", sizeof(pkv_plan_info));
  FIELD(pkv_problem, batch);
  FIELD(pkv_problem, q_len);
  FIELD(pkv_problem, num_q_heads);
  FIELD(pkv_problem, num_kv_heads);
  FIELD(pkv_problem, head_dim);
  FIELD(pkv_problem, page_size);
  FIELD(pkv_problem, num_pages);
  FIELD(pkv_problem, max_pages_per_seq);
  FIELD(pkv_problem, max_kv_len);
  FIELD(pkv_problem, scale);
  FIELD(pkv_problem, causal_offset);
  FIELD(pkv_problem, num_splits);
  FIELD(pkv_problem, mask_stride_b);
  FIELD(pkv_problem, mask_stride_q);
  FIELD(pkv_problem, heads_per_block);
  FIELD(pkv_plan_info, splits);
  FIELD(pkv_plan_info, heads_per_block);
  FIELD(pkv_plan_info, rows_per_block);
  FIELD(pkv_plan_info, matrix_core);
  FIELD(pkv_plan_info, units);
  FIELD(pkv_plan_info, workgroups);
  FIELD(pkv_plan_info, merge_in_kernel);
  FIELD(pkv_plan_info, kernels);
  FIELD(pkv_plan_info, kernel);
  FIELD(pkv_plan_info, paired_heads);
  printf("const %d %d %d %d %d %d %d\n", PKV_MAX_SPLITS, PKV_CAUSAL_LAST, PKV_COUNTER_BYTES, PKV_MAX_FUSED_UNITS,
         PKV_KV_BLHD, PKV_KV_BHLD, PKV_MAX_CONTIGUOUS_KEYS);
  printf("kernels %d %d %d %d\n", PKV_KERNEL_VECTOR, PKV_KERNEL_MATRIX, PKV_KERNEL_SHARED_TILE, PKV_KERNEL_PREFILL);
  printf("status %d %d %d %d %d %d %d %d %d\n", PKV_OK, PKV_ERR_NULL, PKV_ERR_SHAPE, PKV_ERR_UNSUPPORTED,
         PKV_ERR_WORKSPACE, PKV_ERR_ALIGN, PKV_ERR_LAUNCH, PKV_ERR_DEVICE, PKV_ERR_SCRATCH);
  printf("scratch %llu\n", (unsigned long long)PKV_NOALLOC_SCRATCH_BYTES);

  pkv_problem p = decode_problem();
  pkv_plan_info info;
  int splits = -1;
  int rc = pkv_num_splits(&p, 256, &splits);
  printf("num_splits %d %d\n", rc, splits);
  memset(&info, 0, sizeof info);
  print_plan("plan_decode", pkv_plan(&p, 256, &info), &info);

  pkv_problem v = decode_problem();   /* a varlen batch: up to 64 tokens per sequence */
  v.q_len = 64;
  v.causal_offset = PKV_CAUSAL_LAST;
  memset(&info, 0, sizeof info);
  print_plan("plan_varlen", pkv_plan_varlen(&v, 100, 256, &info), &info);

  size_t ob = 0, mb = 0;
  rc = pkv_workspace_bytes(&p, 6, &ob, &mb);
  printf("workspace %d %zu %zu\n", rc, ob, mb);

  /* argument checks, answered on the host */
  printf("err_null_problem %d\n", pkv_plan(NULL, 256, &info));
  printf("err_null_info %d\n", pkv_plan(&p, 256, NULL));
  pkv_problem bad = decode_problem();
  bad.num_kv_heads = 5;
  printf("err_gqa %d\n", pkv_plan(&bad, 256, &info));
  bad = decode_problem();
  bad.head_dim = 96;
  printf("err_head_dim %d\n", pkv_plan(&bad, 256, &info));
  bad = decode_problem();
  bad.page_size = 48;
  printf("err_page %d\n", pkv_plan(&bad, 256, &info));
  bad = decode_problem();
  bad.num_splits = PKV_MAX_SPLITS + 1;
  printf("err_splits %d\n", pkv_plan(&bad, 256, &info));
  printf("err_varlen_tokens %d\n", pkv_plan_varlen(&v, 8 * 64 + 1, 256, &info));
  printf("status_string %s\n", pkv_status_string(PKV_ERR_SHAPE));
  return 0;
}
