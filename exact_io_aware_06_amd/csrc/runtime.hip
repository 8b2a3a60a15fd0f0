// Small HIP runtime helpers shared by the C ABI front end.
#include <hip/hip_runtime.h>

namespace attn {

const char* hip_error_text(int code) {
  return hipGetErrorString(static_cast<hipError_t>(code));
}

}  // namespace attn
