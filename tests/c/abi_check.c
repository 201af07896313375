/* A plain C caller of the library: includes only include/rz.h, links
 * librz.so, and exercises the host-side calls and argument checks (no HIP
 * call is reached: every call here is rejected before, or needs no device).
 * Exit status 0 when every check holds; prints the first failure otherwise. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "rz.h"

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "abi_check: failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                       \
    }                                                                 \
  } while (0)

int main(void) {
  /* a 256-byte aligned, never dereferenced address */
  void* fake = (void*)(uintptr_t)(1u << 20);
  const uint16_t* b16 = (const uint16_t*)fake;
  const int32_t* i32 = (const int32_t*)fake;
  float* f32 = (float*)fake;

  CHECK(rz_version() == ((0 << 16) | (1 << 8)));
  CHECK(strcmp(rz_status_string(RZ_OK), "ok") == 0);
  CHECK(strcmp(rz_status_string(RZ_EWORKSPACE), "workspace too small") == 0);
  CHECK(rz_workspace_bytes(0, 128, 1024) == 0);
  CHECK(rz_workspace_bytes(300, 128, 1024) % 256 == 0);
  CHECK(rz_workspace_bytes_grads(300, 128, 1024) > rz_workspace_bytes(300, 128, 1024));
  CHECK(rz_logits_bytes(300, 128, 1024) > 300u * 1024u * 2u);
  CHECK(rz_vocab_split_begin(151936, 0) == 0);
  CHECK(rz_vocab_split_begin(151936, RZ_VOCAB_SPLITS) == 151936);

  const size_t ws = rz_workspace_bytes(300, 128, 1024);
  /* null, misaligned, bad sizes, short workspace: rejected on the host */
  CHECK(rz_logprob(NULL, b16, 1e-6f, b16, i32, 300, 128, 1024, f32, f32, fake, ws, NULL) ==
        RZ_EINVAL);
  CHECK(rz_logprob(b16 + 4, b16, 1e-6f, b16, i32, 300, 128, 1024, f32, f32, fake, ws, NULL) ==
        RZ_EINVAL);
  CHECK(rz_logprob(b16, b16, 1e-6f, b16, i32, 300, 100, 1024, f32, f32, fake, ws, NULL) ==
        RZ_EUNSUPPORTED);
  CHECK(rz_logprob(b16, b16, 1e-6f, b16, i32, 300, 128, 1024, f32, f32, fake, ws - 1, NULL) ==
        RZ_EWORKSPACE);
  CHECK(rz_backward(b16, b16, 1e-6f, b16, i32, f32, NULL, 300, 128, 1024, f32, fake, ws,
                    NULL) == RZ_EINVAL);
  CHECK(rz_backward_grads(b16, b16, 1e-6f, b16, i32, f32, f32, 300, 128, 1024, NULL, 0, f32,
                          NULL, f32, fake, rz_workspace_bytes_grads(300, 128, 1024),
                          NULL) == RZ_EINVAL);
  CHECK(rz_logprob_noalloc(b16, b16, 1e-6f, b16, i32, 8573, 1536, 151936, f32, NULL, NULL) ==
        RZ_EWORKSPACE);
  puts("abi_check: ok");
  return 0;
}
