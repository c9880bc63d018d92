#!/bin/bash
cd /root/repo/_work
INC="-I../include -I../linear_attention_context_amd/csrc"
FL="--offload-arch=gfx950 -O3 -std=c++17 -fPIC -shared -fvisibility=hidden -Wno-unused-command-line-argument -Xclang -target-feature -Xclang -packed-fp32-ops"
API=../linear_attention_context_amd/csrc/qla_api.cpp
K=../linear_attention_context_amd/csrc/qla_kernels.hip
for t in 0 1 2 3; do
  hipcc $FL $INC -DQLA_M_TOUCH=$t -o lib/libqla_v26t$t.so $API $K > /dev/null 2>&1 &
done
wait
ls lib | grep v26
